// Router: scores, softmax, top-k (plain, group-limited or per head) and gates.
//
// Gating network and top-K selector: "MoE技术演进", section "Adaptive Mixtures of
// Local Experts" (softmax gating equation).  Group-limited selection:
// "MoE技术演进", "DeepSeek-V2" item 3 (pick the best M devices, then top-K inside;
// devices are groups of consecutive experts here).  Per-head selection inside
// a fixed expert partition: "多头 LatentMoE 与 Head Parallel", 方法论 item 2.
// Aux loss: "MoE技术演进", "GShard" item 1.  Balancing bias added to the
// probabilities for selection, its update, and the sequence-wise balance term:
// "MoE技术演进", "DeepSeek-V3" items 1 and 4.  Expert-choice routing (every
// token offers every expert; the experts choose in dispatch): the LocMoE+
// article's router-taxonomy paragraph.
//
// One kernel computes every token's scores, softmax, top-k and gates
// (route_kernel, below); the aux loss and the per-sequence balance statistic
// add small fixed-order reductions when they are asked for.
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ the router kernel
// One launch: scores, softmax, selection and gates of TB tokens of one head
// per block (grid: ceil(T/TB) x H; 256 threads = 4 waves).
//
// Scores.  Wave w owns token group wt = w / WK (MW*16 tokens) and k-group
// wk = w % WK: a contiguous range of the head's d_head columns.  Both MFMA
// operands come straight from global memory into registers: x rows (the A
// fragments) and W_r rows (the B fragments), D k-steps ahead in a register
// ring, so every byte of W_r a block needs is loaded once per token group
// and x is read once.  A float32 router with bf16 activations is split in
// registers into three bf16 planes hi + mid + lo (exact for normal-range
// values), so bf16 x times each plane is exact in float32 and the three
// MFMAs sum to the float32 dot product to float32 accuracy.  The WK partial
// scores of each (token, expert) meet in LDS and are added in wave order.
//
// Selection.  L lanes (a power of two <= 32) per token; lane j owns the
// head's experts j, j+L, ...  Softmax max and sum by butterflies over the L
// lanes (cross-lane moves by DPP).  Where a gate decides an integer result
// (the affinity keep rule, expert choice, the balancing-bias keys) the
// probabilities are evaluated in float64 (exp of the float32 score
// difference, a float64 sum, one division) and rounded to float32 once: the
// float32 gates are then the correctly rounded probabilities up to float64
// rounding, so those decisions are the ones the exactly rounded values give.
// Otherwise they are evaluated in float32.  Top-k: k rounds of a 64-bit (score key, inverted
// index) maximum over the L lanes: larger score first, lower expert index on
// equal scores.  Per block the kernel also writes each expert's probability
// sum over its tokens and its choice count (the aux-loss partials and the
// per-block expert histogram).
struct RouteArgs {
  const void *x;               // [T][ldx] router input; head h reads columns [h*dh, (h+1)*dh)
  const void *w;               // [E][dh] router weights (router dtype)
  const float *bias;           // [E] or NULL
  const float *sel_bias;       // [E] or NULL: balancing bias of the selection keys
  const float *logits_in;      // LOAD: [T][E] final scores
  float *logits_out;           // STORE: [T][E]
  int32_t *topk_idx;           // [T][H*k]  (expert choice: [T][E])
  float *topk_w;
  float *probs;                // [T][E] or NULL: every probability (sequence statistic)
  float *psum;                 // [nbx][E] or NULL: per-block probability sums
  int32_t *hist;               // [nbx][E] or NULL: per-block choice counts
  int T, H, E, Eh, dh, ldx, k, L, Lg, n_groups, topk_groups, renorm, sel_gate, all_experts, load, WT, WK, TB;
  int epl;                     // selection register slots per lane: 1, 2, 4 or ROUTE_EPL
  int exact;                   // probabilities in float64 (they decide the keep rule or the choice)
};

// 8 float32 values -> three bf16 vectors hi, mid, lo with hi + mid + lo == v
// exactly (normal-range values): hi keeps the top 8 significant bits of v
// (truncation), mid the next 8 of the exact remainder v - hi, and lo the
// remainder v - hi - mid, which has at most 8 significant bits left.
__device__ __forceinline__ void split3(const u32x4 &a, const u32x4 &b, u32x4 &hi, u32x4 &mid, u32x4 &lo) {
  const uint32_t u[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = u[i] & 0xFFFF0000u;
    const float r1 = __uint_as_float(u[i]) - __uint_as_float(h[i]);
    m[i] = __float_as_uint(r1) & 0xFFFF0000u;
    l[i] = __float_as_uint(r1 - __uint_as_float(m[i]));  // low 16 bits are zero
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // element 2q in the low half, 2q+1 in the high half
    hi[q] = (h[2 * q] >> 16) | h[2 * q + 1];
    mid[q] = (m[2 * q] >> 16) | m[2 * q + 1];
    lo[q] = (l[2 * q] >> 16) | (l[2 * q + 1] & 0xFFFF0000u);
  }
}

// ---- reductions over an aligned group of L lanes (L a power of two <= 64)
// Level i pairs each lane with one in the other half of its aligned group of
// 2^(i+1) lanes: quad permutations and row mirrors (DPP, no LDS traffic) up
// to 16 lanes, a swizzle (lane ^ 16) for 32, a permute for 64.  A commutative operation applied
// level by level leaves every lane of the group with the same, bitwise
// identical result, in an order fixed by the lane pattern.
template <int LV>
__device__ __forceinline__ uint32_t xlane(uint32_t v) {
  if constexpr (LV == 0) return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  else if constexpr (LV == 1) return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  else if constexpr (LV == 2) return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else if constexpr (LV == 3) return __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false);  // row_mirror
  else if constexpr (LV == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);  // lane ^ 16 (in 32)
  else return (uint32_t)__builtin_amdgcn_ds_bpermute((int)((threadIdx.x ^ 32) & 63) * 4, (int)v);  // lane ^ 32
}
template <int LV> __device__ __forceinline__ float xlane_f(float v) { return __uint_as_float(xlane<LV>(__float_as_uint(v))); }
template <int LV> __device__ __forceinline__ uint64_t xlane_u64(uint64_t v) {
  return ((uint64_t)xlane<LV>((uint32_t)(v >> 32)) << 32) | xlane<LV>((uint32_t)v);
}
template <int LV> __device__ __forceinline__ double xlane_d(double v) {
  return __longlong_as_double((long long)xlane_u64<LV>((uint64_t)__double_as_longlong(v)));
}

__device__ __forceinline__ float lanes_max(float v, int L) {
  if (L >= 2) v = fmaxf(v, xlane_f<0>(v));
  if (L >= 4) v = fmaxf(v, xlane_f<1>(v));
  if (L >= 8) v = fmaxf(v, xlane_f<2>(v));
  if (L >= 16) v = fmaxf(v, xlane_f<3>(v));
  if (L >= 32) v = fmaxf(v, xlane_f<4>(v));
  if (L >= 64) v = fmaxf(v, xlane_f<5>(v));
  return v;
}
__device__ __forceinline__ uint64_t lanes_max_u64(uint64_t v, int L) {
  uint64_t o;
  if (L >= 2) { o = xlane_u64<0>(v); v = o > v ? o : v; }
  if (L >= 4) { o = xlane_u64<1>(v); v = o > v ? o : v; }
  if (L >= 8) { o = xlane_u64<2>(v); v = o > v ? o : v; }
  if (L >= 16) { o = xlane_u64<3>(v); v = o > v ? o : v; }
  if (L >= 32) { o = xlane_u64<4>(v); v = o > v ? o : v; }
  if (L >= 64) { o = xlane_u64<5>(v); v = o > v ? o : v; }
  return v;
}
__device__ __forceinline__ float lanes_sum_f(float v, int L) {
  if (L >= 2) v += xlane_f<0>(v);
  if (L >= 4) v += xlane_f<1>(v);
  if (L >= 8) v += xlane_f<2>(v);
  if (L >= 16) v += xlane_f<3>(v);
  if (L >= 32) v += xlane_f<4>(v);
  if (L >= 64) v += xlane_f<5>(v);
  return v;
}
__device__ __forceinline__ double lanes_sum_d(double v, int L) {
  if (L >= 2) v += xlane_d<0>(v);
  if (L >= 4) v += xlane_d<1>(v);
  if (L >= 8) v += xlane_d<2>(v);
  if (L >= 16) v += xlane_d<3>(v);
  if (L >= 32) v += xlane_d<4>(v);
  if (L >= 64) v += xlane_d<5>(v);
  return v;
}
constexpr int ROUTE_EPL = 8;   // experts per lane at most (E_h <= 256, L <= 64)
constexpr int ROUTE_KMAX = 8;

// The scores of the block's TB tokens, finalised in LDS row-major [TB][Eh]
// at sc: the WK partial sums added in wave order plus the bias (bsh: the
// head's bias in LDS, or NULL), or (LOAD) the given scores; -0.0 folded to
// +0.0; copied out when they are asked for.  Global traffic is coalesced
// rows, the LOAD reads four per thread at a time; sc may alias the first
// partial sums.
__device__ __forceinline__ void route_scores(const RouteArgs &a, const float *part, float *sc, const float *bsh,
                                             int tb0) {
  const int Eh = a.Eh, TB = a.TB, h = blockIdx.y;
  const int nt = min(TB, a.T - tb0);
  const int n = nt * Eh;
  if (a.load) {
    for (int i0 = threadIdx.x; i0 < n; i0 += 4 * 256) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = i0 + u * 256;
        const int tl = idx / Eh, e = idx - tl * Eh;
        v[u] = idx < n ? a.logits_in[(size_t)(tb0 + tl) * a.E + (size_t)h * Eh + e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (i0 + u * 256 < n) sc[i0 + u * 256] = v[u] + 0.0f;
    }
    return;
  }
  for (int idx = threadIdx.x; idx < n; idx += 256) {
    const int tl = idx / Eh, e = idx - tl * Eh;
    float v = part[idx];
    for (int q = 1; q < a.WK; ++q) v += part[(size_t)q * TB * Eh + idx];
    if (bsh) v += bsh[e];
    if (a.logits_out) a.logits_out[(size_t)(tb0 + tl) * a.E + (size_t)h * Eh + e] = v + 0.0f;
    sc[idx] = v + 0.0f;
  }
}

// The head's router bias and selection bias for this thread's expert
// (E_h <= 256 threads), loaded when the block starts so that the loads
// overlap the scores, and stored to LDS (with the choice counts zeroed)
// before the barrier that precedes route_scores.
struct HeadBias {
  float b, sb;
};
__device__ __forceinline__ HeadBias head_bias_load(const RouteArgs &a) {
  HeadBias r{0.f, 0.f};
  const int e = threadIdx.x, h = blockIdx.y;
  if (e < a.Eh) {
    if (a.bias) r.b = a.bias[h * a.Eh + e];
    if (a.sel_bias) r.sb = a.sel_bias[h * a.Eh + e];
  }
  return r;
}
__device__ __forceinline__ void head_bias_store(const RouteArgs &a, const HeadBias &r, int32_t *cnt, float *sbias,
                                                float *bsh) {
  const int e = threadIdx.x;
  if (e < a.Eh) {
    cnt[e] = 0;
    if (sbias) sbias[e] = r.sb;
    if (bsh) bsh[e] = r.b;
  }
}

// The selection phase of route_kernel: the block's TB tokens of head
// blockIdx.y, scores from sc (LDS [TB][Eh]), choices and gates to global
// memory, choice counts into `cnt`, and (when they are asked for) the
// probabilities into sc in place of the scores.
//
// L lanes per token.  Without groups lane j owns experts j, j+L, ...  With
// groups the lanes are dealt to groups: Lg lanes per group (a power of two),
// lane j = g*Lg + r owning experts g*gsz + r, g*gsz + r + Lg, ... of group g,
// so a group's score is a reduction over its own Lg lanes only.  EPL: the
// register slots per lane (at least the most experts a lane owns); the
// unused slots hold -inf scores and zero weights, which change no result.
template <int EPL>
__device__ __forceinline__ void route_select_n(const RouteArgs &a, float *sc, const float *sbias, int32_t *cnt,
                                               int tb0) {
  const int tid = threadIdx.x;
  const int h = blockIdx.y, Eh = a.Eh, TB = a.TB;
  const int L = a.L, Lg = a.Lg, ppb = 256 / L, pr = tid / L, j = tid % L;
  const float NEG = -__builtin_huge_valf();
  const int Ebase = h * Eh;
  const bool grouped = a.n_groups > 0;
  const int gsz = grouped ? Eh / a.n_groups : Eh;
  // this lane's group (grouped) and its experts: e0 + step * i, i < nown
  const int g = grouped ? j / Lg : 0;
  const int e0 = grouped ? g * gsz + j % Lg : j;
  const int step = grouped ? Lg : L;
  const int span = grouped ? (g < a.n_groups ? gsz - j % Lg : 0) : Eh - j;
  const int nown = span > 0 ? (span + step - 1) / step : 0;
  const bool need_p = a.probs || a.psum || a.all_experts || a.sel_bias;
  for (int p0 = 0; p0 < TB; p0 += ppb) {
    const int tl = p0 + pr;
    const int t = tb0 + tl;
    const bool valid = tl < TB && t < a.T;
    float *srow = sc + (valid ? tl : 0) * Eh + e0;
    float lv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) lv[i] = (valid && i < nown) ? srow[step * i] : NEG;
    float m = NEG;
#pragma unroll
    for (int i = 0; i < EPL; ++i) m = fmaxf(m, lv[i]);
    m = lanes_max(m, L);
    // probabilities: in float64, rounded once, where a gate decides an
    // integer result (exact); in float32 otherwise
    float pf[EPL];
    double ex[EPL];  // exp(l - m): float64 (exact), or float32 widened
    double sum;
    if (a.exact) {
      double sd = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ex[i] = (valid && i < nown) ? exp((double)lv[i] - (double)m) : 0.0;
        sd += ex[i];
      }
      sum = lanes_sum_d(sd, L);
#pragma unroll
      for (int i = 0; i < EPL; ++i) pf[i] = (float)(ex[i] / sum);
    } else {
      float exf[EPL];
      float sf = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        exf[i] = (valid && i < nown) ? __expf(lv[i] - m) : 0.0f;
        sf += exf[i];
      }
      sf = lanes_sum_f(sf, L);
      sum = sf;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        ex[i] = exf[i];
        pf[i] = exf[i] / sf;
      }
    }
    if (need_p && valid) {
      // the probabilities replace this lane's scores (read back by the
      // block's copy-out, the aux partials and expert choice)
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (i < nown) srow[step * i] = pf[i];
    }
    if (a.all_experts) {  // expert choice: every expert is a slot; gates are copied out by the block
      if (valid) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (i < nown) atomicAdd(&cnt[e0 + step * i], 1);
      }
      continue;
    }
    // selection keys: the scores, or p + b under the balancing bias
    uint32_t ky[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      ky[i] = score_key((valid && i < nown) ? (sbias ? (pf[i] + sbias[e0 + step * i]) + 0.0f : lv[i]) : NEG);
    bool allowed = true;
    if (grouped) {
      // group score: the largest key of the group, over the group's Lg lanes
      uint32_t gk = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) gk = max(gk, ky[i]);
      uint64_t gkey = (uint64_t)gk;
      for (int o = 0; (1 << o) < Lg; ++o) {  // levels below Lg: max within the group
        uint64_t x2;
        switch (o) {
          case 0: x2 = xlane_u64<0>(gkey); break;
          case 1: x2 = xlane_u64<1>(gkey); break;
          case 2: x2 = xlane_u64<2>(gkey); break;
          case 3: x2 = xlane_u64<3>(gkey); break;
          default: x2 = xlane_u64<4>(gkey); break;
        }
        gkey = x2 > gkey ? x2 : gkey;
      }
      // composite group key: larger score first, lower group on ties; lanes
      // past the last group take no part
      gkey = (g < a.n_groups) ? ((gkey << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g)) : 0ull;
      allowed = false;
      for (int r = 0; r < a.topk_groups; ++r) {
        const uint64_t best = lanes_max_u64(allowed ? 0ull : gkey, L);
        if (gkey == best) allowed = true;
      }
    }
    uint64_t kk[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = e0 + step * i;
      kk[i] = (valid && i < nown && allowed) ? (((uint64_t)ky[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
    }
    // k rounds: the largest remaining key over the token's lanes; the lane
    // holding it records the round
    int rnk[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) rnk[i] = -1;
#pragma unroll
    for (int r = 0; r < ROUTE_KMAX; ++r) {
      if (r >= a.k) break;
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) best = kk[i] > best ? kk[i] : best;
      best = lanes_max_u64(best, L);
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (kk[i] == best) {
          kk[i] = 0;
          rnk[i] = r;
        }
      }
    }
    // gates of the chosen experts, by the lanes that hold them: the
    // probability (+ bias), renormalised by the sum over the chosen
    double gw[EPL], gs = 0.0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      gw[i] = 0.0;
      if (rnk[i] >= 0) {
        gw[i] = a.exact ? ex[i] / sum : (double)pf[i];
        if (sbias && a.sel_gate) gw[i] += (double)sbias[e0 + step * i];
      }
      gs += gw[i];
    }
    if (a.renorm) gs = lanes_sum_d(gs, L);
    if (valid) {
      int32_t *oi = a.topk_idx + (size_t)t * a.H * a.k + (size_t)h * a.k;
      float *ow = a.topk_w + (size_t)t * a.H * a.k + (size_t)h * a.k;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        if (rnk[i] >= 0) {
          const int e = e0 + step * i;
          oi[rnk[i]] = Ebase + e;
          ow[rnk[i]] = (float)(a.renorm ? gw[i] / gs : gw[i]);
          atomicAdd(&cnt[e], 1);
        }
      }
    }
  }
}

// the selection with as few register slots per lane as the launch's lanes need
// (narrow partitions; the staged kernels take the ROUTE_EPL form directly)
__device__ __forceinline__ void route_select(const RouteArgs &a, float *sc, const float *sbias, int32_t *cnt,
                                             int tb0) {
  switch (a.epl) {
    case 1: route_select_n<1>(a, sc, sbias, cnt, tb0); break;
    case 2: route_select_n<2>(a, sc, sbias, cnt, tb0); break;
    case 4: route_select_n<4>(a, sc, sbias, cnt, tb0); break;
    default: route_select_n<ROUTE_EPL>(a, sc, sbias, cnt, tb0); break;
  }
}

// Scores of the wide expert partitions (16*NF >= 64 experts per head, router
// weights in the activation dtype): per 128-byte k-chunk the block stages
// the head's W_r rows (16*NF) and its TB = 16*MW token rows in LDS with
// direct global->LDS loads, each wave instruction filling eight whole
// 128-byte lines (slots XOR-swizzled by row so that the 16 rows one fragment
// read touches fall in distinct banks), three stages deep.  Wave w owns the
// expert fragments w, w+4, w+8, ... for all TB tokens over the whole d_head,
// so every W_r byte is fetched once per block and read from LDS once, and
// the scores need no cross-wave sum.  Writes the unbiased scores to sc.
constexpr int ROUTE_STAGES = 3;

template <typename TE, int NF, int MW> struct StagedGeom {
  static constexpr int ROWS = 16 * NF + 16 * MW;       // W_r rows, then token rows
  static constexpr int NL = (ROWS * 8 + 255) / 256;     // direct loads per thread per stage
  static constexpr int SLOTS = NL * 256;                // 16-byte slots per stage
  static constexpr int NFW = (NF + 3) / 4;              // expert fragments per wave
};

template <typename TE, int NF, int MW>
__device__ __forceinline__ void route_scores_staged(const RouteArgs &a, u32x4 *ring, float *sc, int tb0) {
  using G = StagedGeom<TE, NF, MW>;
  constexpr int EPC = 16 / sizeof(TE);  // elements per 16-byte slot
  constexpr int CH = 8 * EPC;           // elements per 128-byte chunk
  constexpr int EP = 16 * NF;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, cq = lane >> 4;
  const int h = blockIdx.y, Eh = a.Eh;
  const int nch = a.dh / CH;
  const TE *wb = (const TE *)a.w + (size_t)h * Eh * a.dh;
  const TE *xb = (const TE *)a.x + (size_t)h * a.dh;
  // source of each staged slot (chunk 0): W_r rows past E_h and padding
  // slots read row 0, token rows past T read the last token
  const TE *src[G::NL];
#pragma unroll
  for (int i = 0; i < G::NL; ++i) {
    const int sl = i * 256 + tid, row = sl >> 3, q = (sl & 7) ^ (row & 7);
    if (row >= EP && row < G::ROWS) {
      const int t = min(a.T - 1, tb0 + row - EP);
      src[i] = xb + (size_t)t * a.ldx + q * EPC;
    } else {
      const int e = (row < Eh) ? row : 0;
      src[i] = wb + (size_t)e * a.dh + q * EPC;
    }
  }
  auto issue = [&](int c, int st) {
#pragma unroll
    for (int i = 0; i < G::NL; ++i) load_lds16(src[i] + (size_t)c * CH, ring + st * G::SLOTS + i * 256 + wv * 64);
  };
  f32x4 acc[MW][G::NFW];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int f = 0; f < G::NFW; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  // fragment rows are multiples of 16 plus l16, so the swizzle is l16 & 7
  auto compute = [&](int st) {
    const u32x4 *r = ring + st * G::SLOTS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int sw = (ks * 4 + cq) ^ (l16 & 7);
      u32x4 xa[MW];
#pragma unroll
      for (int i = 0; i < MW; ++i) xa[i] = r[(EP + i * 16 + l16) * 8 + sw];
#pragma unroll
      for (int f = 0; f < G::NFW; ++f) {
        const int fr = wv + 4 * f;
        if (fr < NF) {
          const u32x4 wbv = r[(fr * 16 + l16) * 8 + sw];
#pragma unroll
          for (int i = 0; i < MW; ++i) acc[i][f] = mma16(xa[i], wbv, acc[i][f], TE());
        }
      }
    }
  };
#pragma unroll
  for (int c = 0; c < ROUTE_STAGES - 1; ++c)
    if (c < nch) issue(c, c);
  for (int c = 0; c < nch; ++c) {
    // chunk c landed (the loads of the chunks after it, if all were issued, may
    // still be in flight) and this wave's reads of the stage refilled next are
    // done; a fence-free barrier, so those later chunks stay in flight
    if (c + ROUTE_STAGES - 2 < nch) wait_vmcnt<(ROUTE_STAGES - 2) * G::NL>(); else wait_vmcnt0();
    wait_lgkmcnt0();
    barrier_nofence();
    if (c + ROUTE_STAGES - 1 < nch) issue(c + ROUTE_STAGES - 1, (c + ROUTE_STAGES - 1) % ROUTE_STAGES);
    compute(c % ROUTE_STAGES);
  }
  // acc[i][f][v] = score of token i*16 + 4*cq + v, expert (wv + 4f)*16 + l16
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int f = 0; f < G::NFW; ++f) {
      const int e = (wv + 4 * f) * 16 + l16;
      if (wv + 4 * f < NF && e < Eh) {
#pragma unroll
        for (int v = 0; v < 4; ++v) sc[(i * 16 + 4 * cq + v) * Eh + e] = acc[i][f][v];
      }
    }
}

// Per-block expert statistics, tokens added in order (aux-loss partials and
// the choice histogram); probabilities (sequence statistic) and the
// expert-choice slots copied out in rows.  sc holds the probabilities.
__device__ __forceinline__ void route_block_stats(const RouteArgs &a, const float *sc, const int32_t *cnt, int tb0) {
  const int tid = threadIdx.x, Eh = a.Eh, TB = a.TB, h = blockIdx.y;
  const int nt = min(TB, a.T - tb0);
  for (int e = tid; e < Eh; e += 256) {
    if (a.psum) {
      float acc = 0.f;
      for (int q = 0; q < nt; ++q) acc += sc[(size_t)q * Eh + e];
      a.psum[(size_t)blockIdx.x * a.E + (size_t)h * Eh + e] = acc;
    }
    if (a.hist) a.hist[(size_t)blockIdx.x * a.E + (size_t)h * Eh + e] = cnt[e];
  }
  if (a.probs || a.all_experts) {
    for (int idx = tid; idx < nt * Eh; idx += 256) {
      const int tl = idx / Eh, e = idx - tl * Eh;
      const size_t g = (size_t)(tb0 + tl) * a.E + (size_t)h * Eh + e;
      if (a.probs) a.probs[g] = sc[idx];
      if (a.all_experts) {  // one head: slot e of token t is expert e, its gate p
        a.topk_idx[g] = e;
        a.topk_w[g] = sc[idx];
      }
    }
  }
}

// Register budget of one route_kernel instantiation: V VGPRs per k-step of
// operands and D k-steps in flight.  Four waves per SIMD (128 registers,
// 64 for the operand ring) for the narrowest bf16 tiles, whose launches hold
// many small blocks; two (256, 128 for the ring) for most; one (512, 200 for
// the ring) for the widest tiles (ten or more expert fragments x token
// fragments).
template <typename TIN, typename TW, int NF, int MW> struct RouteRegs {
  static constexpr int EPC = 16 / sizeof(TIN);       // activation elements per 16 bytes
  static constexpr int NWL = EPC * sizeof(TW) / 16;  // 16-byte W loads per lane per k-step
  static constexpr int V = 4 * (MW + NF * NWL);
  static constexpr int OCC = NF * MW >= 10 ? 1 : ((NF * MW <= 2 && NWL == 1) ? 4 : 2);
  static constexpr int BUDGET = OCC == 1 ? 200 : (OCC == 2 ? 128 : 64);  // VGPRs for the operand ring
  static constexpr int D = (BUDGET / V) < 2 ? 2 : ((BUDGET / V) > 8 ? 8 : (BUDGET / V));
};

// EPLK > 0: the selection with that many register slots per lane only (the
// launch's own form: a kernel holding every form is sized for the largest)
template <typename TIN, typename TW, int NPL, int NF, int MW, bool ST, int EPLK = 0>
__global__ __launch_bounds__(256, (ST ? 2 : RouteRegs<TIN, TW, NF, MW>::OCC)) void route_kernel(RouteArgs a) {
  // LDS: [WK][TB][Eh] partial scores (then scores, probabilities), [Eh]
  // counts, [Eh] bias, and (staged scores) the chunk ring
  extern __shared__ float rsm[];
  if constexpr (ST) {
    const int Eh = a.Eh, TB = a.TB, tb0 = blockIdx.x * TB;
    float *sc = rsm;
    int32_t *cnt = (int32_t *)(sc + (size_t)TB * Eh);
    float *sbias = a.sel_bias ? (float *)(cnt + Eh) : nullptr;
    float *bsh = a.bias ? (float *)(cnt + 2 * Eh) : nullptr;
    u32x4 *ring = (u32x4 *)(rsm + align_up((size_t)TB * Eh + 3 * Eh, 4));
    const HeadBias hb = head_bias_load(a);
    if (!a.load) route_scores_staged<TIN, NF, MW>(a, ring, sc, tb0);
    head_bias_store(a, hb, cnt, sbias, bsh);
    __syncthreads();
    route_scores(a, sc, sc, bsh, tb0);  // one set of scores (WK == 1): bias, or the loaded scores
    __syncthreads();
    route_select_n<ROUTE_EPL>(a, sc, sbias, cnt, tb0);  // wide partitions: at least 4 experts per lane
    __syncthreads();
    route_block_stats(a, sc, cnt, tb0);
    return;
  } else {
  using RR = RouteRegs<TIN, TW, NF, MW>;
  constexpr int EPC = RR::EPC;
  constexpr int KSTEP = 4 * EPC;                     // k per MFMA call (4 lane groups x 16 bytes)
  constexpr int NWL = RR::NWL;
  constexpr int D = RR::D;                           // k-steps in flight
  static_assert(NPL == 1 || (NPL == 3 && NWL == 2), "three planes split a float32 router for bf16 inputs");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, cq = lane >> 4;
  const int h = blockIdx.y, Eh = a.Eh, TB = a.TB;
  const int tb0 = blockIdx.x * TB;
  float *part = rsm;
  int32_t *cnt = (int32_t *)(rsm + (size_t)(a.load ? 1 : a.WK) * TB * Eh);
  float *sbias = a.sel_bias ? (float *)(cnt + Eh) : nullptr;  // the head's selection bias
  float *bsh = a.bias ? (float *)(cnt + 2 * Eh) : nullptr;     // the head's router bias
  const HeadBias hb = head_bias_load(a);

  if (!a.load) {
    const int wt = wv / a.WK, wk = wv % a.WK;
    if (wt < a.WT) {
      const int ns = a.dh / KSTEP;
      const int s0 = (int)((long)wk * ns / a.WK), s1 = (int)((long)(wk + 1) * ns / a.WK);
      const TIN *xb = (const TIN *)a.x + (size_t)h * a.dh + cq * EPC;
      const TW *wb = (const TW *)a.w + (size_t)h * Eh * a.dh + cq * EPC;
      const TIN *xrow[MW];
#pragma unroll
      for (int i = 0; i < MW; ++i) {
        const int t = min(a.T - 1, tb0 + wt * MW * 16 + i * 16 + l16);
        xrow[i] = xb + (size_t)t * a.ldx;
      }
      // rows past E_h read row 0 (their scores are never stored): every load
      // is unconditional, so the compiler's wait counts stay exact
      const TW *wrow[NF];
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int e = f * 16 + l16;
        wrow[f] = wb + (size_t)(e < Eh ? e : 0) * a.dh;
      }
      f32x4 acc[MW][NF];
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 xr[D][MW], wr[D][NF][NWL];
      auto load = [&](int s, int d) {
        const size_t ko = (size_t)s * KSTEP;
#pragma unroll
        // x streams through once: non-temporal, so it does not evict W_r from L2
        for (int i = 0; i < MW; ++i) xr[d][i] = __builtin_nontemporal_load((const u32x4 *)(xrow[i] + ko));
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int q = 0; q < NWL; ++q) wr[d][f][q] = *(const u32x4 *)(wrow[f] + ko + q * (16 / sizeof(TW)));
      };
      auto compute = [&](int d) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if constexpr (NPL == 3) {
            u32x4 hi, mid, lo;
            split3(wr[d][f][0], wr[d][f][1], hi, mid, lo);
#pragma unroll
            for (int i = 0; i < MW; ++i) {
              acc[i][f] = mma16(xr[d][i], hi, acc[i][f], uint16_t());
              acc[i][f] = mma16(xr[d][i], mid, acc[i][f], uint16_t());
              acc[i][f] = mma16(xr[d][i], lo, acc[i][f], uint16_t());
            }
          } else {
#pragma unroll
            for (int i = 0; i < MW; ++i) acc[i][f] = mma16(xr[d][i], wr[d][f][0], acc[i][f], TW());
          }
        }
      };
      // register ring: slot d holds logical step l + d.  A chunk of D steps
      // is computed while the next chunk's loads (clamped to the last step)
      // are in flight; the last chunk (1..D steps) issues no loads.  Logical
      // step l is d_head step s0 + (l + rot) mod n: the blocks an XCD runs
      // at once start at different columns, so they do not all ask the same
      // L2 lines of W_r for the same columns at the same time.
      const int n = s1 - s0;
      if (n > 0) {
        const int rot = (int)(((long)(blockIdx.x >> 3) % 32) * n / 32);
        auto phys = [&](int l) { const int q = l + rot; return s0 + (q >= n ? q - n : q); };
#pragma unroll
        for (int d = 0; d < D; ++d) load(phys(min(d, n - 1)), d);
        int l = 0;
        for (; l + D < n; l += D) {
#pragma unroll
          for (int d = 0; d < D; ++d) {
            compute(d);
            load(phys(min(l + D + d, n - 1)), d);
            // keep the steps in order: the scheduler would otherwise hoist
            // later steps' work and wait for their loads too early
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
        for (int d = 0; d < D; ++d)
          if (l + d < n) compute(d);
      }
      // acc[i][f][v] = score of token 4*cq + v of fragment i, expert f*16 + l16
      float *pw = part + (size_t)wk * TB * Eh;
#pragma unroll
      for (int i = 0; i < MW; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int e = f * 16 + l16;
          if (e < Eh) {
#pragma unroll
            for (int v = 0; v < 4; ++v) pw[(size_t)(wt * MW * 16 + i * 16 + 4 * cq + v) * Eh + e] = acc[i][f][v];
          }
        }
    }
  }
  head_bias_store(a, hb, cnt, sbias, bsh);
  __syncthreads();

  route_scores(a, part, part, bsh, tb0);
  __syncthreads();
  if constexpr (EPLK > 0) route_select_n<EPLK>(a, part, sbias, cnt, tb0);
  else route_select(a, part, sbias, cnt, tb0);
  __syncthreads();
  route_block_stats(a, part, cnt, tb0);
  }
}

// aux = sum_e (sum_b psum[b][e] / T) * (sum_b hist[b][e]) / T, block sums in order
__global__ void route_aux_kernel(const float *__restrict__ psum, const int32_t *__restrict__ hist, int nblocks,
                                 int E, int T, float *__restrict__ aux) {
  __shared__ float red[256];
  float v = 0.f;
  for (int e = threadIdx.x; e < E; e += 256) {
    float me = 0.f;
    long ce = 0;
    for (int b = 0; b < nblocks; ++b) {
      me += psum[(size_t)b * E + e];
      ce += hist[(size_t)b * E + e];
    }
    v += (me / (float)T) * ((float)ce / (float)T);
  }
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *aux = red[0];
}

// Per-sequence balance statistic, two passes.  Pass 1: one block per chunk of
// SEQ_CH tokens inside one sequence: column sums of p over the chunk (tokens in
// order) and the chunk's choice counts (integer LDS atomics, order-free).
// Pass 2: one block per sequence adds its chunks in order and reduces
// sum_e (c_e / L) (P_e / L) by a fixed tree.
constexpr int SEQ_CH = 32;

__global__ __launch_bounds__(256) void route_seq_part_kernel(const float *__restrict__ probs,
                                                             const int32_t *__restrict__ topk_idx, int E, int K,
                                                             int L, int nch, float *__restrict__ psum,
                                                             int32_t *__restrict__ pcnt) {
  extern __shared__ int cnt[];  // [E]
  const int tid = threadIdx.x;
  const int sq = blockIdx.x / nch, ch = blockIdx.x % nch;
  const long t0 = (long)sq * L + (long)ch * SEQ_CH;
  const int nt = min(SEQ_CH, L - ch * SEQ_CH);
  for (int e = tid; e < E; e += 256) cnt[e] = 0;
  __syncthreads();
  for (int i = tid; i < nt * K; i += 256) atomicAdd(&cnt[topk_idx[t0 * K + i]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    float P = 0.f;
    for (int t = 0; t < nt; ++t) P += probs[(size_t)(t0 + t) * E + e];
    psum[(size_t)blockIdx.x * E + e] = P;
    pcnt[(size_t)blockIdx.x * E + e] = cnt[e];
  }
}

__global__ __launch_bounds__(256) void route_seq_kernel(const float *__restrict__ psum,
                                                        const int32_t *__restrict__ pcnt, int E, int L, int nch,
                                                        float *__restrict__ seq_loss) {
  __shared__ float red[256];
  __shared__ float gp[256];
  __shared__ int gc[256];
  const int tid = threadIdx.x;
  const size_t b0 = (size_t)blockIdx.x * nch;
  float v = 0.f;
  if (E <= 128) {
    // G groups of E threads split the chunks; the groups' sums are added in order
    const int G = 256 / E, g = tid / E, e = tid % E;
    if (g < G) {
      const int c0 = (int)((long)nch * g / G), c1 = (int)((long)nch * (g + 1) / G);
      float P = 0.f;
      int c = 0;
      for (int ch = c0; ch < c1; ++ch) {
        P += psum[(b0 + ch) * E + e];
        c += pcnt[(b0 + ch) * E + e];
      }
      gp[g * E + e] = P;
      gc[g * E + e] = c;
    }
    __syncthreads();
    if (tid < E) {
      float P = 0.f;
      long c = 0;
      for (int q = 0; q < G; ++q) {
        P += gp[q * E + tid];
        c += gc[q * E + tid];
      }
      v = ((float)c / (float)L) * (P / (float)L);
    }
  } else {
    for (int e = tid; e < E; e += 256) {
      float P = 0.f;
      long c = 0;
      for (int ch = 0; ch < nch; ++ch) {
        P += psum[(b0 + ch) * E + e];
        c += pcnt[(b0 + ch) * E + e];
      }
      v += ((float)c / (float)L) * (P / (float)L);
    }
  }
  red[tid] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  if (tid == 0) seq_loss[blockIdx.x] = red[0];
}

// Balancing-bias update, one block per head: b_e += gamma * sign(N_h - n_e E_h)
// with N_h the head's total load (integer comparison).
__global__ __launch_bounds__(256) void sel_bias_update_kernel(const int32_t *__restrict__ load, float *sel_bias,
                                                              int Eh, float gamma) {
  __shared__ long long red[256];
  const int tid = threadIdx.x, h = blockIdx.x;
  long long v = 0;
  for (int e = tid; e < Eh; e += 256) v += load[(size_t)h * Eh + e];
  red[tid] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const long long tot = red[0];
  for (int e = tid; e < Eh; e += 256) {
    const long long n = (long long)load[(size_t)h * Eh + e] * Eh;
    const float step = n > tot ? -1.f : (n < tot ? 1.f : 0.f);
    sel_bias[(size_t)h * Eh + e] = sel_bias[(size_t)h * Eh + e] + gamma * step;
  }
}

// ------------------------------------------------------------------ host launchers
// fragment counts with an instantiated kernel: 16*NF >= E_h rows of W_r per head
static int round_nf(int nf) {
  static const int sup[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16};
  for (int v : sup)
    if (v >= nf) return v;
  return -1;
}

RouteGeom route_geometry(const Shape &s) {
  RouteGeom g{};
  g.nf = round_nf((s.Eh + 15) / 16);
  g.nplanes = (s.router_f32 && !s.act_f32) ? 3 : 1;
  const int kstep = s.act_f32 ? 16 : 32;
  const int ns = s.dh / kstep;
  // several heads, or a short d_head: four token groups of 16 per block, each
  // over the whole d_head; otherwise one token group split over the four
  // waves along d_head, with two 16-token fragments when the batch holds
  // enough tokens for 256 such blocks
  g.st = (g.nf >= 4 && g.nplanes == 1) ? 1 : 0;
  if (g.st) {
    // wide partitions: staged chunks, the waves split the experts
    g.wt = 1; g.wk = 1;
    g.mw = (!s.act_f32 && s.T >= 2 * 256 * 16) ? 2 : 1;
  } else if (s.H > 1 || ns < 16) {
    g.wt = 4; g.wk = 1; g.mw = 1;
  } else {
    g.wt = 1; g.wk = 4;
    g.mw = (!s.act_f32 && g.nf <= 10 && s.T >= 2 * 256 * 16) ? 2 : 1;
  }
  g.tb = g.wt * g.mw * 16;
  g.nbx = (s.T + g.tb - 1) / g.tb;
  // selection lanes per token
  if (s.n_groups > 0) {
    // Lg lanes per group (at most ROUTE_EPL experts each), the groups side by side
    const int gsz = s.Eh / s.n_groups;
    g.Lg = 1;
    while (g.Lg * ROUTE_EPL < gsz) g.Lg *= 2;
    g.L = 1;
    while (g.L < s.n_groups * g.Lg) g.L *= 2;
    g.epl = (gsz + g.Lg - 1) / g.Lg;
  } else {
    // at most ROUTE_EPL experts per lane; more lanes (up to one per expert)
    // while the block's tokens still fit in one pass
    g.Lg = 0;
    g.L = 1;
    while (g.L < 64 && g.L * ROUTE_EPL < s.Eh) g.L *= 2;
    while (g.L < 64 && g.L < s.Eh && 2 * g.L * g.tb <= 256) g.L *= 2;
    g.epl = (s.Eh + g.L - 1) / g.L;
  }
  return g;
}

// LDS: the partial scores [WK][TB][E_h] (one set with LOAD), the choice
// counts [E_h], the head's selection bias [E_h] and router bias [E_h]
static size_t route_lds_bytes(const Shape &s, const RouteGeom &g, bool load) {
  if (g.st) {  // scores [TB][E_h], counts, biases, then the ring of staged chunks
    const size_t nl = ((size_t)(16 * g.nf + 16 * g.mw) * 8 + 255) / 256;
    return align_up((size_t)g.tb * s.Eh + 3 * s.Eh, 4) * 4 + (load ? 0 : ROUTE_STAGES * nl * 256 * 16);
  }
  return ((size_t)(load ? 1 : g.wk) * g.tb * s.Eh + 3 * s.Eh) * 4;
}

size_t route_hist_offset(const Shape &s) {
  return align_up((size_t)route_geometry(s).nbx * s.E * 4, 256);  // past the per-block probability sums
}

size_t route_stats_bytes(const Shape &s) { return 2 * route_hist_offset(s); }

size_t route_ws_bytes(const Shape &s) {
  size_t b = route_stats_bytes(s);  // per-block probability sums and choice counts
  if (s.seq_len > 0) {
    const size_t nb = (size_t)(s.T / s.seq_len) * ((s.seq_len + SEQ_CH - 1) / SEQ_CH);
    b += align_up((size_t)s.T * s.E * 4, 256);  // probabilities
    b += 2 * align_up(nb * s.E * 4, 256);       // chunk sums and counts
  }
  return b;
}

#define LAUNCH_CHECK() do { if (int rc_ = launch_status("route")) return rc_; } while (0)

template <typename TIN, typename TW, int NPL, int NF, int MW, bool ST, int EPLK = 0>
static int launch_one(const RouteArgs &a, const RouteGeom &g, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((route_kernel<TIN, TW, NPL, NF, MW, ST, EPLK>), dim3((unsigned)g.nbx, (unsigned)a.H), dim3(256),
                     lds, st, a);
  return 0;
}

// narrow partitions (NF <= 3; up to 6 for the three-plane router): per-wave
// operand rings; wide ones: staged chunks
template <typename TIN, typename TW, int NPL, int NF>
static int launch_route_t(const RouteArgs &a, const RouteGeom &g, size_t lds, hipStream_t st) {
  constexpr bool kST = NPL == 1 && NF >= 4;
  if constexpr (sizeof(TIN) == 2 && (kST || NF <= 10)) {
    if (g.mw == 2) return launch_one<TIN, TW, NPL, NF, 2, kST>(a, g, lds, st);
  }
  // one expert fragment per head (E_h <= 16: many heads, or few experts):
  // kernels with the launch's own selection form (measured on the multi-head
  // workload: 89 instead of 124 VGPRs, router 27.9 -> 27.0 us cold; a form
  // held to 64 VGPRs for eight waves per SIMD, four k-steps in flight, took
  // 43.8 us)
  if constexpr (!kST && NF == 1) {
    if (g.epl == 1) return launch_one<TIN, TW, NPL, NF, 1, kST, 1>(a, g, lds, st);
    if (g.epl == 2) return launch_one<TIN, TW, NPL, NF, 1, kST, 2>(a, g, lds, st);
    if (g.epl == 4) return launch_one<TIN, TW, NPL, NF, 1, kST, 4>(a, g, lds, st);
  }
  return launch_one<TIN, TW, NPL, NF, 1, kST>(a, g, lds, st);
}

template <typename TIN, typename TW, int NPL>
static int launch_route_nf(const RouteArgs &a, const RouteGeom &g, size_t lds, hipStream_t st) {
  switch (g.nf) {
    case 1: return launch_route_t<TIN, TW, NPL, 1>(a, g, lds, st);
    case 2: return launch_route_t<TIN, TW, NPL, 2>(a, g, lds, st);
    case 3: return launch_route_t<TIN, TW, NPL, 3>(a, g, lds, st);
    case 4: return launch_route_t<TIN, TW, NPL, 4>(a, g, lds, st);
    case 5: return launch_route_t<TIN, TW, NPL, 5>(a, g, lds, st);
    case 6: return launch_route_t<TIN, TW, NPL, 6>(a, g, lds, st);
    default:
      if constexpr (NPL == 1) {
        switch (g.nf) {
          case 8: return launch_route_t<TIN, TW, NPL, 8>(a, g, lds, st);
          case 10: return launch_route_t<TIN, TW, NPL, 10>(a, g, lds, st);
          case 12: return launch_route_t<TIN, TW, NPL, 12>(a, g, lds, st);
          case 16: return launch_route_t<TIN, TW, NPL, 16>(a, g, lds, st);
        }
      }
      return -2;
  }
}

bool route_supported(const Shape &s) {
  const RouteGeom g = route_geometry(s);
  // the three-plane (fp32 router, bf16 activations) form is instantiated up
  // to 6 fragments (E_h <= 96)
  if (g.nplanes == 3 && g.nf > 6) return false;
  if (route_lds_bytes(s, g, false) > 160 * 1024) return false;
  return g.nf > 0 && g.epl <= ROUTE_EPL && g.L <= 64;
}

int launch_route(const Shape &s, const void *x, const void *w_router, const float *bias, const float *sel_bias,
                 float *logits, int mode, int32_t *topk_idx, float *topk_w, float *aux_loss, float *seq_loss,
                 void *ws, hipStream_t st, int32_t *hist_out) {
  const RouteGeom g = route_geometry(s);
  char *p = (char *)ws;
  float *psum = (float *)p;
  int32_t *hist = (int32_t *)(p + route_hist_offset(s));
  p += route_stats_bytes(s);
  float *probs = nullptr, *spsum = nullptr;
  int32_t *pcnt = nullptr;
  const int nseq = s.seq_len > 0 ? s.T / s.seq_len : 0, nch = s.seq_len > 0 ? (s.seq_len + SEQ_CH - 1) / SEQ_CH : 0;
  if (seq_loss) {
    probs = (float *)p;
    p += align_up((size_t)s.T * s.E * 4, 256);
    spsum = (float *)p;
    p += align_up((size_t)nseq * nch * s.E * 4, 256);
    pcnt = (int32_t *)p;
  }
  const bool load = mode == 2;
  const bool aux = aux_loss != nullptr;
  RouteArgs a{};
  a.x = x; a.w = w_router; a.bias = load ? nullptr : bias;
  a.sel_bias = s.expert_choice ? nullptr : sel_bias;
  a.logits_in = load ? logits : nullptr;
  a.logits_out = (mode == 1) ? logits : nullptr;
  a.topk_idx = topk_idx; a.topk_w = topk_w; a.probs = probs;
  a.psum = aux ? psum : nullptr;
  a.hist = hist_out ? hist_out : (aux ? hist : nullptr);
  a.T = s.T; a.H = s.H; a.E = s.E; a.Eh = s.Eh; a.dh = s.dh; a.ldx = s.H * s.dh; a.k = s.k; a.L = g.L; a.Lg = g.Lg;
  a.exact = (s.drop == DROP_AFFINITY || s.expert_choice || (sel_bias && !s.expert_choice)) ? 1 : 0;
  a.n_groups = s.n_groups; a.topk_groups = s.topk_groups; a.renorm = s.renorm; a.sel_gate = s.sel_gate;
  a.all_experts = s.expert_choice; a.load = load ? 1 : 0; a.WT = g.wt; a.WK = g.wk; a.TB = g.tb;
  a.epl = g.epl <= 1 ? 1 : (g.epl <= 2 ? 2 : (g.epl <= 4 ? 4 : ROUTE_EPL));
  const size_t lds = route_lds_bytes(s, g, load);
  int rc;
  if (s.act_f32) rc = launch_route_nf<float, float, 1>(a, g, lds, st);
  else if (g.nplanes == 3) rc = launch_route_nf<uint16_t, float, 3>(a, g, lds, st);
  else rc = launch_route_nf<uint16_t, uint16_t, 1>(a, g, lds, st);
  if (rc) return rc;
  LAUNCH_CHECK();
  if (aux) {
    hipLaunchKernelGGL(route_aux_kernel, dim3(1), dim3(256), 0, st, psum, a.hist, g.nbx, s.E, s.T, aux_loss);
    LAUNCH_CHECK();
  }
  if (seq_loss) {
    hipLaunchKernelGGL(route_seq_part_kernel, dim3((unsigned)(nseq * nch)), dim3(256), (size_t)s.E * 4, st, probs,
                       topk_idx, s.E, s.K, s.seq_len, nch, spsum, pcnt);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(route_seq_kernel, dim3((unsigned)nseq), dim3(256), 0, st, spsum, pcnt, s.E, s.seq_len, nch,
                       seq_loss);
    LAUNCH_CHECK();
  }
  return 0;
}

int launch_sel_bias_update(const Shape &s, const int32_t *load, float *sel_bias, float gamma, hipStream_t st) {
  hipLaunchKernelGGL(sel_bias_update_kernel, dim3((unsigned)s.H), dim3(256), 0, st, load, sel_bias, s.Eh, gamma);
  return launch_status("selection bias update");
}

}  // namespace moe
