// Backward through the content-aware erase (CARVE notes, section 2.2) on gfx950.
//
// Once the forward has run, every content period p (L tokens) has a fixed gate
// b = sigmoid(b_x + z_p), z_p = U2 (U1 m_{p-1}); the chunk gradients are those of the
// token-only rule with that b, the erase gradient taken directly w.r.t. the gate's
// pre-activation (dx = dlog a (1 - b) = db b (1 - b)).  What couples the periods is the
// mean output: m_{p-1} feeds z_p, so period p's gate gradient dx gives
//   dz_p = sum_t dx_t,  dU2 += dz_p r_p^T (r_p = U1 m_{p-1}),  dr = U2^T dz_p,
//   dU1 += dr m_{p-1}^T,  dm_{p-1} = U1^T dr,
// and dm_{p-1} / L is added to the output gradient of every token of period p-1
// (period 0's dm goes to m0).  The library runs the periods in reverse; these
// kernels are the per-period pieces around the token-only backward kernels.
// The file also holds the logit-space epilogue of the backward for gates given as
// pre-activations (d f, d A, d tau).
#include "carve_chunk.h"
#include "content_gate.h"

namespace carve {

// b = sigmoid(b_x + z_p) for every token, the same expression as the forward's gate
__global__ __launch_bounds__(256) void content_gates_kernel(ContentBwdArgs a, const float* b_x, float* bmat) {
  const size_t n4 = (size_t)a.B * a.H * a.T * a.D / 4;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    const size_t e = 4 * i;
    const int k = (int)(e % a.D);
    const size_t row = e / a.D;                      // (bh, t)
    const int t = (int)(row % a.T);
    const size_t bh = row / a.T;
    const float* z = a.z_all + (bh * a.NP + t / a.L) * a.D + k;
    const f32x4 x = *reinterpret_cast<const f32x4*>(b_x + e);
    f32x4 b;
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = 1.f / (1.f + fexp(-(x[j] + z[j])));
    *reinterpret_cast<f32x4*>(bmat + e) = b;
  }
}

// dO' = dO + g (g per head and value column) for the tokens of period p
template <typename T>
__global__ __launch_bounds__(256) void add_grad_mean_kernel(ContentBwdArgs a, const T* dO, T* dOp) {
  const int bh = blockIdx.x;
  const int t0 = a.p * a.L, t1 = min(t0 + a.L, a.T);
  const size_t base = ((size_t)bh * a.T + t0) * a.D;
  const int n4 = (t1 - t0) * a.D / 4;
  const float* g = a.g + (size_t)bh * a.D;
  for (int i = threadIdx.x; i < n4; i += blockDim.x) {
    const int col = (4 * i) % a.D;
    const f32x4 x = load4f(dO + base + 4 * i);
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + col);
    store4(dOp + base + 4 * i, x + gv);
  }
}

// One workgroup per head runs the gate backward of period p (content_gate.h).
template <typename T, int D>
__global__ __launch_bounds__(256) void content_gate_bwd_kernel(ContentBwdArgs a, const T* dO, T* dOp) {
  extern __shared__ float lds[];
  content_gate_body<T, D, 256>(a, blockIdx.x, dO, dOp, lds);
}

// g = dm_out / (tokens of the last period), or 0
__global__ __launch_bounds__(256) void init_grad_mean_kernel(ContentBwdArgs a, const float* dm_out) {
  const size_t n = (size_t)a.B * a.H * a.D;
  const float inv = 1.f / (float)(a.T - (a.NP - 1) * a.L);
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    a.g[i] = dm_out ? dm_out[i] * inv : 0.f;
}

// out[h][i] = sum over the batch of part[b * H + h][i]
__global__ __launch_bounds__(256) void sum_over_batch_kernel(const float* part, float* out, int B, int H, int n) {
  const size_t total = (size_t)H * n;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
    const size_t h = i / n, j = i % n;
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += part[((size_t)b * H + h) * n + j];
    out[i] = s;
  }
}

// ------------------------------------------------------------ gate pre-activations
// d/df = d/dlog g * (-A sigmoid(f + tau)) in place over the buffer holding d/dlog g,
// with per-(sequence, token block) column sums of d/df (-> d tau) and of
// d/dlog g * (-softplus(f + tau)) (-> d A).  One workgroup per (b*H + h, block of
// kLogitBlock tokens); thread t owns column t % D and every (256 / D)-th token.
constexpr int kLogitBlock = 256;
__global__ __launch_bounds__(256) void logit_grads_kernel(LogitGradArgs a) {
  __shared__ float pa[256], pt[256];
  const int bh = blockIdx.x, tb = blockIdx.y, tid = threadIdx.x, D = a.D, h = bh % a.H;
  const int k = tid % D, part = tid / D, nparts = 256 / D;
  const float A = a.A[h * D + k], tau = a.tau[h * D + k];
  const int t0 = tb * kLogitBlock, t1 = min(t0 + kLogitBlock, a.T);
  // tokens t0 + part + nparts j, eight at a time: the loads of a batch are issued before
  // its stores (the compiler cannot move a load past a store to df, which it must assume
  // may alias f); the sums run in token order
  float sa = 0.f, st = 0.f;
  for (int tb = t0 + part; tb < t1; tb += 8 * nparts) {
    float fv[8], dv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t i = ((size_t)bh * a.T + min(tb + nparts * u, t1 - 1)) * D + k;
      fv[u] = a.f[i];
      dv[u] = a.df[i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = tb + nparts * u;
      if (t < t1) {
        const float y = fv[u] + tau;
        const float df = -dv[u] * A * sigmoidf(y);
        a.df[((size_t)bh * a.T + t) * D + k] = df;
        st += df;
        sa -= dv[u] * softplusf(y);
      }
    }
  }
  pa[tid] = sa;
  pt[tid] = st;
  __syncthreads();
  if (tid < D) {
    float s1 = 0.f, s2 = 0.f;
    for (int pp = 0; pp < nparts; ++pp) {
      s1 += pa[pp * D + tid];
      s2 += pt[pp * D + tid];
    }
    const size_t o = ((size_t)bh * gridDim.y + tb) * D + tid;
    a.partA[o] = s1;
    a.partT[o] = s2;
  }
}

// outX[h][k] = sum over the batch and token blocks of partX[(b*H + h) * nblk + tb][k], for
// X = A (threads 0 .. H*D-1) and X = tau (the next H*D); summed in the order b, tb, with
// the loads issued eight at a time
__global__ __launch_bounds__(256) void sum_heads_kernel(const float* partA, const float* partT, float* outA,
                                                        float* outT, int B, int H, int nblk, int D) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * H * D) return;
  const bool isA = i < H * D;
  if (!isA) i -= H * D;
  const float* part = isA ? partA : partT;
  const int h = i / D, k = i % D, n = B * nblk;
  float s = 0.f;
  for (int j0 = 0; j0 < n; j0 += 8) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + u, n - 1), b = j / nblk, tb = j % nblk;
      x[u] = part[(((size_t)b * H + h) * nblk + tb) * D + k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < n) s += x[u];
  }
  (isA ? outA : outT)[i] = s;
}

hipError_t launch_logit_grads(const LogitGradArgs& a, float* dA, float* dtau, hipStream_t st) {
  const int nblk = (a.T + kLogitBlock - 1) / kLogitBlock;
  hipLaunchKernelGGL(logit_grads_kernel, dim3(a.B * a.H, nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned g = (unsigned)((2 * a.H * a.D + 255) / 256);
  hipLaunchKernelGGL(sum_heads_kernel, dim3(g), dim3(256), 0, st, a.partA, a.partT, dA, dtau, a.B, a.H, nblk, a.D);
  return hipGetLastError();
}

size_t logit_partials_bytes(int B, int H, int T, int D) {
  return 2 * (size_t)B * H * ((T + kLogitBlock - 1) / kLogitBlock) * D * sizeof(float);
}

static unsigned grid_for(size_t n, unsigned cap = 4096) {
  const size_t g = (n + 255) / 256;
  return (unsigned)(g < cap ? (g ? g : 1) : cap);
}

hipError_t launch_content_gates(const ContentBwdArgs& a, const float* b_x, float* bmat, hipStream_t st) {
  hipLaunchKernelGGL(content_gates_kernel, dim3(grid_for((size_t)a.B * a.H * a.T * a.D / 4)), dim3(256), 0, st, a,
                     b_x, bmat);
  return hipGetLastError();
}

hipError_t launch_add_grad_mean(const ContentBwdArgs& a, int dtype, const void* dO, void* dOp, hipStream_t st) {
  if (dtype)
    hipLaunchKernelGGL(add_grad_mean_kernel<bf16>, dim3(a.B * a.H), dim3(256), 0, st, a,
                       reinterpret_cast<const bf16*>(dO), reinterpret_cast<bf16*>(dOp));
  else
    hipLaunchKernelGGL(add_grad_mean_kernel<float>, dim3(a.B * a.H), dim3(256), 0, st, a,
                       reinterpret_cast<const float*>(dO), reinterpret_cast<float*>(dOp));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t gate_bwd_launch_d(const ContentBwdArgs& a, const void* dO, void* dOp, hipStream_t st) {
  const size_t lds = sizeof(float) * content_gate_lds_floats(D, 256, a.U1 ? a.R : 0);
  auto kern = content_gate_bwd_kernel<T, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)(sizeof(float) * content_gate_lds_floats(D, 256, 64)));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(256), lds, st, a, reinterpret_cast<const T*>(dO), reinterpret_cast<T*>(dOp));
  return hipGetLastError();
}
template <typename T>
static hipError_t gate_bwd_launch(const ContentBwdArgs& a, const void* dO, void* dOp, hipStream_t st) {
  return a.D == 128 ? gate_bwd_launch_d<T, 128>(a, dO, dOp, st) : gate_bwd_launch_d<T, 64>(a, dO, dOp, st);
}

hipError_t launch_content_gate_bwd(const ContentBwdArgs& a, int dtype, const void* dO, void* dOp, hipStream_t st) {
  return dtype ? gate_bwd_launch<bf16>(a, dO, dOp, st) : gate_bwd_launch<float>(a, dO, dOp, st);
}

hipError_t launch_init_grad_mean(const ContentBwdArgs& a, const float* dm_out, hipStream_t st) {
  hipLaunchKernelGGL(init_grad_mean_kernel, dim3(grid_for((size_t)a.B * a.H * a.D)), dim3(256), 0, st, a, dm_out);
  return hipGetLastError();
}

hipError_t launch_sum_over_batch(const float* part, float* out, int B, int H, int n, hipStream_t st) {
  hipLaunchKernelGGL(sum_over_batch_kernel, dim3(grid_for((size_t)H * n)), dim3(256), 0, st, part, out, B, H, n);
  return hipGetLastError();
}

}  // namespace carve
