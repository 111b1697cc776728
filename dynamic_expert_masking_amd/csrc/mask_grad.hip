// Mask-router backward of the BEAM layer: the loss value L_reg and the
// straight-through gradient with respect to the mask router.
//
// Method: BEAM page on aitrends.kr ("BEAM: Dynamic MoE 라우팅을 위한 Binary
// Expert Activation Masking"), training strategy in the method paragraph:
// L = L_lm + alpha L_bal + beta L_reg, L_reg = (1/K) sum_{i in TK} |m_hat_i|,
// and the straight-through estimator passes the gradient of m_hat through the
// binarisation (also the ai-feeds.com summary, method section, binarisation
// and STE).  Over a batch L_reg is the mean over tokens.  With
// y = sum_k g_k m_k E_k(x) and dm/dm_hat := 1:
//
//   dL/dm_hat_k = g_k <dL/dy, E_k(x)> + beta / (T K)      (m_hat > 0)
//   dL/dz_k     = dL/dm_hat_k * m_hat_k (1 - m_hat_k),  m_hat = sigmoid(z)
//   dL/dWm[e]   = sum over candidates (t, k) of expert e of dL/dz_k x_t
//   dL/db_m[e]  = sum over the same candidates of dL/dz_k
//
// The caller's routing ran in all-pairs mode: every top-K candidate has an
// expert output row O[slot_pos[t][k]] (the layer's dtype), gates[t][k] holds the unmasked
// g, zsel[t][k] the mask logit, and the pairs are in expert-major order.
#include "beam_internal.h"
#include "device_common.h"

namespace beam {

// Sum over the workgroup's 256 threads in a fixed order (deterministic).
__device__ __forceinline__ float block_sum256(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f32(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

// One workgroup per token: dot products <dL/dy_t, O[pair]> over D for the
// token's K candidates, then dL/dz of each candidate (written at its pair
// position) and the token's sum of m_hat.
template <bool BF16>
__global__ __launch_bounds__(256) void k_mask_grad_pairs(const void* __restrict__ dy, int T, int D,
                                                         int K, float beta,
                                                         const float* __restrict__ gates,
                                                         const float* __restrict__ zsel,
                                                         const int32_t* __restrict__ slot_pos,
                                                         const void* __restrict__ o,
                                                         float* __restrict__ dz,
                                                         float* __restrict__ lreg_tok) {
  __shared__ float red[4];
  const int t = blockIdx.x;
  float msum = 0.f;
  for (int k = 0; k < K; ++k) {
    const int pos = slot_pos[size_t(t) * K + k];
    float part = 0.f;
    for (int d = 4 * threadIdx.x; d < D; d += 4 * 256) {
      const float4 g4 = ld4_f32<BF16>(dy, size_t(t) * D + d);
      const float4 o4 = ld4_f32<BF16>(o, size_t(pos) * D + d);
      part += (g4.x * o4.x + g4.y * o4.y) + (g4.z * o4.z + g4.w * o4.w);
    }
    const float dot = block_sum256(part, red);
    const float z = zsel[size_t(t) * K + k];
    const float mh = 1.f / (1.f + expf(-z));
    msum += mh;
    if (threadIdx.x == 0) {
      const float dmh = gates[size_t(t) * K + k] * dot + beta / (float(T) * float(K));
      dz[pos] = dmh * mh * (1.f - mh);
    }
  }
  if (threadIdx.x == 0) lreg_tok[t] = msum;
}

// dL/dWm[e][d..d+3] for the 4 columns of this thread: the expert's pairs are
// rows expert_off[e] .. expert_off[e+1] of the pair order (tokens ascending),
// added in that order, 8 pairs' loads in flight at a time.  Workgroup (e, 0)
// also writes dL/db_m[e]; workgroup (0, 0) writes L_reg.
template <bool BF16>
__global__ __launch_bounds__(256) void k_mask_grad_wm(const void* __restrict__ x, int T, int D, int K,
                                                      const int32_t* __restrict__ expert_off,
                                                      const int32_t* __restrict__ perm_token,
                                                      const float* __restrict__ dz,
                                                      const float* __restrict__ lreg_tok,
                                                      float* __restrict__ dwm,
                                                      float* __restrict__ dbm,
                                                      float* __restrict__ lreg) {
  __shared__ float red[4];
  const int e = blockIdx.x;
  const int d = 4 * (blockIdx.y * 256 + threadIdx.x);
  const int p0 = expert_off[e], p1 = expert_off[e + 1];
  if (d < D) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = p0; q0 < p1; q0 += 8) {
      float w[8];
      float4 xv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = min(q0 + u, p1 - 1);
        w[u] = q0 + u < p1 ? dz[q] : 0.f;
        xv[u] = ld4_f32<BF16>(x, size_t(perm_token[q]) * D + d);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc.x += w[u] * xv[u].x;
        acc.y += w[u] * xv[u].y;
        acc.z += w[u] * xv[u].z;
        acc.w += w[u] * xv[u].w;
      }
    }
    *reinterpret_cast<float4*>(dwm + size_t(e) * D + d) = acc;
  }
  if (blockIdx.y == 0 && dbm != nullptr && threadIdx.x == 0) {
    float s = 0.f;
    for (int q = p0; q < p1; ++q) s += dz[q];
    dbm[e] = s;
  }
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    float part = 0.f;
    for (int t = threadIdx.x; t < T; t += 256) part += lreg_tok[t];
    const float s = block_sum256(part, red);
    if (threadIdx.x == 0) *lreg = s / (float(T) * float(K));
  }
}

hipError_t launch_mask_grad(const beam_moe_layer& L, const void* x, const void* dy, int32_t T,
                            float beta, float* dwm, float* dbm, float* lreg, const Ptrs& p,
                            hipStream_t s) {
  const bool bf = L.dtype == BEAM_BF16;
  prof_before("mask_grad_pairs", s);
  if (bf)
    hipLaunchKernelGGL(k_mask_grad_pairs<true>, dim3(unsigned(T)), dim3(256), 0, s, dy, T, L.D, L.K,
                       beta, p.gates, p.zsel, p.slot_pos, p.o, p.dz, p.lreg_tok);
  else
    hipLaunchKernelGGL(k_mask_grad_pairs<false>, dim3(unsigned(T)), dim3(256), 0, s, dy, T, L.D, L.K,
                       beta, p.gates, p.zsel, p.slot_pos, p.o, p.dz, p.lreg_tok);
  prof_after(s);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const dim3 g(unsigned(L.E), unsigned((L.D + 1023) / 1024));
  prof_before("mask_grad_wm", s);
  if (bf)
    hipLaunchKernelGGL(k_mask_grad_wm<true>, g, dim3(256), 0, s, x, T, L.D, L.K, p.expert_off,
                       p.perm_token, p.dz, p.lreg_tok, dwm, dbm, lreg);
  else
    hipLaunchKernelGGL(k_mask_grad_wm<false>, g, dim3(256), 0, s, x, T, L.D, L.K, p.expert_off,
                       p.perm_token, p.dz, p.lreg_tok, dwm, dbm, lreg);
  prof_after(s);
  return hipGetLastError();
}

}  // namespace beam
