// Layer backward: the elementwise, permutation and router kernels (the
// products run on the grouped GEMM, gemm.hip).
//
// Gradients of <dy, y> + lam * l_aux with the forward's decisions held fixed,
// by the chain rule through the definitions the forward follows: y_t = x_t +
// s_t + sum_kept g_{t,j} F_e(x_t) ("MoE技术演进", "DeepSeekMoE" items 1-2,
// "GShard" item 3); F_e = W2 (SiLU(W1 v) * W3 v) ("大语言模型并行策略（七）：专家
// 并行", "MoE 模型的参数量分析"); g = softmax(W_r x + b) at the chosen experts,
// optionally renormalised ("MoE技术演进", "Adaptive Mixtures of Local Experts"
// gating equation, "DeepSeekMoE" item 1); l_aux = sum_e m_e c_e / S ("GShard"
// item 1).  Every reduction runs in a fixed order (bit-reproducible).
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

__global__ void zero_f32_kernel(float *p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0.f;
}

// ---------------------------------------------------------------- per kept row
// dg[a] = <dy_t, y_perm_r> and dY_r = g_a * dy_t for row r holding assignment
// a = t*K + j.  One wave per row; dg of dropped assignments stays 0.
template <typename TA>
__global__ __launch_bounds__(256) void bwd_rows_kernel(const TA *__restrict__ dy, const TA *__restrict__ y_perm,
                                                       const float *__restrict__ gates,
                                                       const int32_t *__restrict__ src_of,
                                                       const int32_t *__restrict__ offsets, int E, int K, int dh,
                                                       long ld_dy, TA *__restrict__ dY, float *__restrict__ dg) {
  constexpr int EPC = 16 / sizeof(TA);
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= offsets[E]) return;
  const int a = src_of[r], t = a / K;
  const float g = gates[a];
  const u32x4 *s = (const u32x4 *)(dy + (size_t)t * ld_dy);
  const u32x4 *yp = (const u32x4 *)(y_perm + (size_t)r * dh);
  u32x4 *o = (u32x4 *)(dY + (size_t)r * dh);
  float dot = 0.f;
  for (int c = lane; c < dh / EPC; c += 64) {
    const u32x4 vs = s[c], vy = yp[c];
    u32x4 vo;
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s0 = bf16_to_f32((uint16_t)(vs[q] & 0xFFFFu)), s1 = bf16_to_f32((uint16_t)(vs[q] >> 16));
        const float y0 = bf16_to_f32((uint16_t)(vy[q] & 0xFFFFu)), y1 = bf16_to_f32((uint16_t)(vy[q] >> 16));
        dot += s0 * y0;
        dot += s1 * y1;
        vo[q] = (uint32_t)f32_to_bf16(g * s0) | ((uint32_t)f32_to_bf16(g * s1) << 16);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float s0 = __uint_as_float(vs[q]);
        dot += s0 * __uint_as_float(vy[q]);
        vo[q] = __float_as_uint(g * s0);
      }
    }
    o[c] = vo;
  }
  dot = group_sum_fixed(dot, WAVE);
  if (lane == 0) dg[a] = dot;
}

// ---------------------------------------------------------------- expert padding
// poff[e] = sum_{e' < e} roundup(counts[e'], 64): expert e's rows occupy
// columns [poff[e], poff[e] + counts[e]) of the transposed activations, the
// rest of its 64-aligned range is zero.  One block.
__global__ __launch_bounds__(1024) void bwd_poff_kernel(const int32_t *__restrict__ offsets, int E,
                                                        int32_t *__restrict__ poff) {
  __shared__ int s[1024];
  const int tid = threadIdx.x, per = (E + 1023) / 1024;
  int sum = 0, loc[8];
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    const int v = e < E ? (offsets[e + 1] - offsets[e] + 63) / 64 * 64 : 0;
    loc[i] = v;
    sum += v;
  }
  s[tid] = sum;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int u = tid >= o ? s[tid - o] : 0;
    __syncthreads();
    s[tid] += u;
    __syncthreads();
  }
  int run = s[tid] - sum;
  for (int i = 0; i < per && i < 8; ++i) {
    const int e = tid * per + i;
    if (e < E) poff[e] = run;
    run += loc[i];
  }
  if (tid == 1023) poff[E] = s[1023];
}

// pmap_r[j] = row r held by padded column j (or -1); pmap_x[j] = its token
__global__ void bwd_pmap_kernel(const int32_t *__restrict__ offsets, const int32_t *__restrict__ poff,
                                const int32_t *__restrict__ src_of, int E, int K, long npad,
                                int32_t *__restrict__ pmap_r, int32_t *__restrict__ pmap_x) {
  for (long j = blockIdx.x * (long)blockDim.x + threadIdx.x; j < npad; j += (long)gridDim.x * blockDim.x) {
    int r = -1;
    if (j < poff[E]) {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (poff[mid] <= j) lo = mid; else hi = mid - 1;
      }
      const int rr = offsets[lo] + (int)(j - poff[lo]);
      if (rr < offsets[lo + 1]) r = rr;
    }
    pmap_r[j] = r;
    pmap_x[j] = r >= 0 ? src_of[r] / K : -1;
  }
}

// ---------------------------------------------------------------- transpose
// dst[b][c][j] = source row j's column (coff + c), for c < ncols, j < njcols:
//   rmap: source row rmap[j] (zero when -1); else row j when j < nvalid (zero after).
// Tiles of 64 columns x 64 rows through LDS, 16-byte global accesses both ways.
template <typename TA>
__global__ __launch_bounds__(256) void transpose_kernel(const TA *__restrict__ src, long ld_src, long bs_src,
                                                        const int32_t *__restrict__ rmap, long nvalid, long njcols,
                                                        int ncols, int coff, TA *__restrict__ dst, long ld_dst,
                                                        long bs_dst) {
  constexpr int EPC = 16 / sizeof(TA), CH = 64 / EPC;  // 16-byte chunks per 64 elements
  __shared__ TA tile[64][64 + EPC];
  const long j0 = (long)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  src += (size_t)blockIdx.z * bs_src;
  dst += (size_t)blockIdx.z * bs_dst;
  for (int i = threadIdx.x; i < 64 * CH; i += 256) {
    const int jj = i / CH, ch = i % CH;
    const long j = j0 + jj;
    long row = -1;
    if (j < njcols) row = rmap ? (long)rmap[j] : (j < nvalid ? j : -1);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row >= 0 && c0 + ch * EPC < ncols) v = *(const u32x4 *)(src + (size_t)row * ld_src + coff + c0 + ch * EPC);
    const TA *pv = (const TA *)&v;
#pragma unroll
    for (int q = 0; q < EPC; ++q) tile[jj][ch * EPC + q] = pv[q];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * CH; i += 256) {
    const int cc = i / CH, ch = i % CH;
    if (c0 + cc >= ncols || j0 + ch * EPC >= njcols) continue;
    u32x4 v;
    TA *pv = (TA *)&v;
#pragma unroll
    for (int q = 0; q < EPC; ++q) pv[q] = tile[ch * EPC + q][cc];
    *(u32x4 *)(dst + (size_t)(c0 + cc) * ld_dst + j0 + ch * EPC) = v;
  }
}

// ---------------------------------------------------------------- router
// dl[t][e] = p_e (dp_e - sum_e' p_e' dp_e'), p = softmax(logits_t); dp from the
// gate gradients (renormalised: (dg_j - sum dg g) / P at the chosen experts)
// plus lam * demand_e / T^2 (aux loss).  One wave per token.
__global__ __launch_bounds__(256) void router_bwd_kernel(const float *__restrict__ logits,
                                                         const int32_t *__restrict__ topk_idx,
                                                         const float *__restrict__ gates,
                                                         const float *__restrict__ dg,
                                                         const int32_t *__restrict__ demand, int T, int E, int k,
                                                         int renorm, float lam, float *__restrict__ dl) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (t >= T) return;
  const float *l = logits + (size_t)t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
  m = wave_max(m, WAVE);
  float z = 0.f;
  for (int e = lane; e < E; e += 64) z += __expf(l[e] - m);
  z = group_sum_fixed(z, WAVE);
  // chosen experts: P = sum p, S = sum dg * g
  float P = 0.f, sdg = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = topk_idx[(size_t)t * k + j];
    P += __expf(l[e] - m) / z;
    sdg += dg[(size_t)t * k + j] * gates[(size_t)t * k + j];
  }
  const float invT2 = 1.0f / ((float)T * (float)T);
  // dp_e for this lane's experts, then sum p * dp
  float spdp = 0.f;
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(l[e] - m) / z;
    float dp = lam * (float)demand[e] * invT2;
    for (int j = 0; j < k; ++j)
      if (topk_idx[(size_t)t * k + j] == e) dp += renorm ? (dg[(size_t)t * k + j] - sdg) / P : dg[(size_t)t * k + j];
    spdp += p * dp;
  }
  spdp = group_sum_fixed(spdp, WAVE);
  for (int e = lane; e < E; e += 64) {
    const float p = __expf(l[e] - m) / z;
    float dp = lam * (float)demand[e] * invT2;
    for (int j = 0; j < k; ++j)
      if (topk_idx[(size_t)t * k + j] == e) dp += renorm ? (dg[(size_t)t * k + j] - sdg) / P : dg[(size_t)t * k + j];
    dl[(size_t)t * E + e] = p * (dp - spdp);
  }
}

// dW_r[e][c] = sum_t dl[t][e] x[t][c] (float32, t ascending); block y == 0
// also writes dbias[e] = sum_t dl[t][e].  A block owns 64 columns and all E.
template <typename TX>
__global__ __launch_bounds__(512) void router_wgrad_kernel(const float *__restrict__ dl, const TX *__restrict__ x,
                                                           long ldx, int T, int E, int d, float *__restrict__ dw,
                                                           float *__restrict__ dbias) {
  constexpr int TC = 32;         // tokens per staged chunk
  __shared__ float sdl[TC][257];
  __shared__ float sx[TC][64];
  const int c0 = blockIdx.x * 64, tid = threadIdx.x, c = tid & 63, eg = tid >> 6;  // 8 expert groups
  float acc[32], accb[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = accb[i] = 0.f;
  for (int t0 = 0; t0 < T; t0 += TC) {
    const int nt = min(TC, T - t0);
    for (int i = tid; i < TC * E; i += 512) {
      const int tt = i / E, e = i % E;
      sdl[tt][e] = tt < nt ? dl[(size_t)(t0 + tt) * E + e] : 0.f;
    }
    for (int i = tid; i < TC * 64; i += 512) {
      const int tt = i / 64, cc = i % 64;
      sx[tt][cc] = (tt < nt && c0 + cc < d) ? Elem<TX>::to_f32(x[(size_t)(t0 + tt) * ldx + c0 + cc]) : 0.f;
    }
    __syncthreads();
    for (int tt = 0; tt < nt; ++tt) {
      const float xv = sx[tt][c];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int e = eg + 8 * i;
        if (e < E) {
          acc[i] += sdl[tt][e] * xv;
          accb[i] += sdl[tt][e];
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int e = eg + 8 * i;
    if (e < E && c0 + c < d) dw[(size_t)e * d + c0 + c] = acc[i];
    if (e < E && blockIdx.x == 0 && c == 0 && dbias) dbias[e] = accb[i];
  }
}

// ---------------------------------------------------------------- input gradient
// dx[t][c] = [dy[t][c]] + [dxs[t][c]] + sum_j dXr[row_of[t][j]][c] + sum_e dl[t][e] W_r[e][c],
// float32 in that order, rounded once.
template <typename TA, typename TR>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const TA *__restrict__ dy, const TA *__restrict__ dxs,
                                                     const TA *__restrict__ dXr, const int32_t *__restrict__ row_of,
                                                     const float *__restrict__ dl, const TR *__restrict__ w_r, int T,
                                                     int d, int K, int E, int residual, TA *__restrict__ dx) {
  const long n = (long)T * d;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const int t = (int)(i / d), c = (int)(i % d);
    float s = residual ? Elem<TA>::to_f32(dy[i]) : 0.f;
    if (dxs) s += Elem<TA>::to_f32(dxs[i]);
    for (int j = 0; j < K; ++j) {
      const int r = row_of[(size_t)t * K + j];
      if (r >= 0) s += Elem<TA>::to_f32(dXr[(size_t)r * d + c]);
    }
    for (int e = 0; e < E; ++e) s += dl[(size_t)t * E + e] * Elem<TR>::to_f32(w_r[(size_t)e * d + c]);
    dx[i] = Elem<TA>::from_f32(s);
  }
}

// ---------------------------------------------------------------- launchers
template <typename TA>
static int transpose_t(const void *src, long ld_src, long bs_src, const int32_t *rmap, long nvalid, long njcols,
                       int ncols, int coff, void *dst, long ld_dst, long bs_dst, int batches, hipStream_t st) {
  if (njcols <= 0 || ncols <= 0 || batches <= 0) return 0;
  dim3 grid((unsigned)((njcols + 63) / 64), (unsigned)((ncols + 63) / 64), (unsigned)batches);
  hipLaunchKernelGGL((transpose_kernel<TA>), grid, dim3(256), 0, st, (const TA *)src, ld_src, bs_src, rmap, nvalid,
                     njcols, ncols, coff, (TA *)dst, ld_dst, bs_dst);
  return launch_status("transpose");
}

int launch_transpose(bool f32, const void *src, long ld_src, long bs_src, const int32_t *rmap, long nvalid,
                     long njcols, int ncols, int coff, void *dst, long ld_dst, long bs_dst, int batches,
                     hipStream_t st) {
  return f32 ? transpose_t<float>(src, ld_src, bs_src, rmap, nvalid, njcols, ncols, coff, dst, ld_dst, bs_dst,
                                  batches, st)
             : transpose_t<uint16_t>(src, ld_src, bs_src, rmap, nvalid, njcols, ncols, coff, dst, ld_dst, bs_dst,
                                     batches, st);
}

int launch_bwd_rows(const Shape &s, const void *dy, const void *y_perm, const float *gates, const int32_t *src_of,
                    const int32_t *offsets, void *dY, float *dg, hipStream_t st) {
  const long tk = (long)s.T * s.K;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)std::min<long>((tk + 255) / 256, 4096)), dim3(256), 0, st, dg,
                     tk);
  if (int rc = launch_status("zero gate gradients")) return rc;
  if (s.R_max == 0) return 0;
  const unsigned grid = (unsigned)((s.R_max + 3) / 4);
  if (s.act_f32)
    hipLaunchKernelGGL((bwd_rows_kernel<float>), dim3(grid), dim3(256), 0, st, (const float *)dy,
                       (const float *)y_perm, gates, src_of, offsets, s.E, s.K, s.dh, (long)s.d, (float *)dY, dg);
  else
    hipLaunchKernelGGL((bwd_rows_kernel<uint16_t>), dim3(grid), dim3(256), 0, st, (const uint16_t *)dy,
                       (const uint16_t *)y_perm, gates, src_of, offsets, s.E, s.K, s.dh, (long)s.d, (uint16_t *)dY,
                       dg);
  return launch_status("backward rows");
}

int launch_bwd_pad(const Shape &s, const int32_t *offsets, const int32_t *src_of, int32_t *poff, int32_t *pmap_r,
                   int32_t *pmap_x, long npad, hipStream_t st) {
  hipLaunchKernelGGL(bwd_poff_kernel, dim3(1), dim3(1024), 0, st, offsets, s.E, poff);
  if (int rc = launch_status("expert padding")) return rc;
  if (npad <= 0) return 0;
  hipLaunchKernelGGL(bwd_pmap_kernel, dim3((unsigned)std::min<long>((npad + 255) / 256, 8192)), dim3(256), 0, st,
                     offsets, poff, src_of, s.E, s.K, npad, pmap_r, pmap_x);
  return launch_status("padding map");
}

int launch_router_bwd(const Shape &s, const float *logits, const int32_t *topk_idx, const float *gates,
                      const float *dg, const int32_t *demand, float lam, const void *x, float *dl, float *dw_router,
                      float *dbias, hipStream_t st) {
  hipLaunchKernelGGL(router_bwd_kernel, dim3((unsigned)((s.T + 3) / 4)), dim3(256), 0, st, logits, topk_idx, gates,
                     dg, demand, s.T, s.E, s.K, s.renorm, lam, dl);
  if (int rc = launch_status("router backward")) return rc;
  const unsigned grid = (unsigned)((s.d + 63) / 64);
  if (s.act_f32)
    hipLaunchKernelGGL((router_wgrad_kernel<float>), dim3(grid), dim3(512), 0, st, dl, (const float *)x, (long)s.d,
                       s.T, s.E, s.d, dw_router, dbias);
  else
    hipLaunchKernelGGL((router_wgrad_kernel<uint16_t>), dim3(grid), dim3(512), 0, st, dl, (const uint16_t *)x,
                       (long)s.d, s.T, s.E, s.d, dw_router, dbias);
  return launch_status("router weight gradient");
}

__global__ void set_kwin_kernel(int32_t *kwin, int tpad) {
  if (threadIdx.x == 0) {
    kwin[0] = 0;
    kwin[1] = tpad;
  }
}

int launch_set_kwin(int32_t *kwin, int tpad, hipStream_t st) {
  hipLaunchKernelGGL(set_kwin_kernel, dim3(1), dim3(64), 0, st, kwin, tpad);
  return launch_status("k window");
}

int launch_bwd_dx(const Shape &s, const void *dy, const void *dxs, const void *dXr, const int32_t *row_of,
                  const float *dl, const void *w_router, void *dx, hipStream_t st) {
  const long n = (long)s.T * s.d;
  const unsigned grid = (unsigned)std::min<long>((n + 255) / 256, 65536);
  if (s.act_f32) {
    hipLaunchKernelGGL((bwd_dx_kernel<float, float>), dim3(grid), dim3(256), 0, st, (const float *)dy,
                       (const float *)dxs, (const float *)dXr, row_of, dl, (const float *)w_router, s.T, s.d, s.K,
                       s.E, s.residual, (float *)dx);
  } else if (s.router_f32) {
    hipLaunchKernelGGL((bwd_dx_kernel<uint16_t, float>), dim3(grid), dim3(256), 0, st, (const uint16_t *)dy,
                       (const uint16_t *)dxs, (const uint16_t *)dXr, row_of, dl, (const float *)w_router, s.T, s.d,
                       s.K, s.E, s.residual, (uint16_t *)dx);
  } else {
    hipLaunchKernelGGL((bwd_dx_kernel<uint16_t, uint16_t>), dim3(grid), dim3(256), 0, st, (const uint16_t *)dy,
                       (const uint16_t *)dxs, (const uint16_t *)dXr, row_of, dl, (const uint16_t *)w_router, s.T,
                       s.d, s.K, s.E, s.residual, (uint16_t *)dx);
  }
  return launch_status("input gradient");
}

}  // namespace moe
