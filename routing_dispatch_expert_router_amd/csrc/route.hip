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
// Two kernels.  route_logits: a split-K MFMA product of a token tile with the
// head's router weights (staged in LDS, shared by the block's 4 waves), writing
// float32 partial scores [KSPLIT][T][E].  route_select: L lanes per
// (token, head) sum the partials in a fixed order, add the bias, and do
// softmax, group selection, top-k and gates in registers.
#include "common.h"
#include "launch.h"

namespace moe {

// ------------------------------------------------------------------ W_r f32 -> 3 bf16 planes
// hi + mid + lo == w exactly for normal-range values, so x(bf16) * plane
// products are exact in float32 and the MFMA sum approximates the float32 dot.
__global__ void route_split_w_kernel(const float *__restrict__ w, uint16_t *__restrict__ planes,
                                     int E, int Epad, int d, int H, int Eh) {
  // planes: [H][3][Epad][d]; w: [E][d]; head h owns rows h*Eh..
  long total = (long)H * Epad * d;
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < total; i += (long)gridDim.x * blockDim.x) {
    int k = (int)(i % d);
    long r = i / d;
    int e = (int)(r % Epad);
    int h = (int)(r / Epad);
    float v = (e < Eh) ? w[(long)(h * Eh + e) * d + k] : 0.0f;
    uint16_t hi = f32_to_bf16(v);
    float r1 = v - bf16_to_f32(hi);
    uint16_t mid = f32_to_bf16(r1);
    float r2 = r1 - bf16_to_f32(mid);
    uint16_t lo = f32_to_bf16(r2);
    long base = ((long)h * 3 * Epad + e) * d + k;
    planes[base] = hi;
    planes[base + (long)Epad * d] = mid;
    planes[base + 2L * Epad * d] = lo;
  }
}

// ------------------------------------------------------------------ logits (MFMA)
// grid (ceil(T/TB), H, KSPLIT), block 256.  TB = 64*MW tokens; wave w owns
// tokens [w*16*MW, (w+1)*16*MW) of the tile.  The head's W rows (NPL planes x
// NF*16 rows, rows past E_h read row 0 and are never stored) are staged per
// 128-byte k-chunk in LDS with global_load_lds (XOR-swizzled 16-byte slots,
// two stages); x goes straight into MFMA fragments, loaded one chunk ahead.
template <typename TIN, typename TW, int NF, int NPL, int MW>
__global__ __launch_bounds__(256) void route_logits_kernel(
    const TIN *__restrict__ x, const TW *__restrict__ w, float *__restrict__ part,
    int T, int E, int Eh, int dh, int ldx, int kchunk_per_split, long w_head_stride, long w_plane_stride) {
  constexpr int EPC = 16 / sizeof(TIN);            // elements per 16 bytes
  constexpr int CHUNK = 8 * EPC;                   // elements per 128-byte row chunk
  constexpr int ROWS = NPL * NF * 16;
  constexpr int NWI = (ROWS * 8 + 255) / 256;      // W load instructions per thread per chunk
  constexpr int STAGE = NWI * 256;                 // slots per stage (padded to whole instructions)
  constexpr int NL = NWI + 2 * MW;                 // vector-memory instructions per thread per chunk
  __shared__ u32x4 lds[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int h = blockIdx.y, ks = blockIdx.z;
  const int tok0 = blockIdx.x * (64 * MW);
  const int Epad = NF * 16;
  const int nchunks = dh / CHUNK;
  const int c0 = ks * kchunk_per_split;
  const int c1 = min(nchunks, c0 + kchunk_per_split);
  const TW *wh = w + (size_t)h * w_head_stride;
  const TIN *xh = x + (size_t)h * dh;
  const int cq = lane >> 4, l16 = lane & 15;

  // W source of each staged slot (row 0 for padding rows and padding slots)
  uint32_t woff[NWI];
#pragma unroll
  for (int i = 0; i < NWI; ++i) {
    const int sl = i * 256 + tid;
    const int r = sl >> 3, q = (sl & 7) ^ (r & 7);
    const int pl = r / Epad, e = r - pl * Epad;
    woff[i] = (sl < ROWS * 8 && e < Eh) ? (uint32_t)(pl * w_plane_stride + (long)e * dh + q * (16 / sizeof(TW)))
                                        : (uint32_t)(q * (16 / sizeof(TW)));
  }
  int arow[MW];
#pragma unroll
  for (int i = 0; i < MW; ++i) arow[i] = min(T - 1, tok0 + wv * 16 * MW + i * 16 + l16);

  auto issue = [&](int c, int st, u32x4 (&xa)[MW][2]) {
#pragma unroll
    for (int i = 0; i < NWI; ++i)
      load_lds16(wh + woff[i] + (size_t)c * (8 * 16 / sizeof(TW)), lds + st * STAGE + i * 256 + wv * 64);
#pragma unroll
    for (int i = 0; i < MW; ++i) {
      const u32x4 *src = reinterpret_cast<const u32x4 *>(xh + (size_t)arow[i] * ldx + (size_t)c * CHUNK);
      xa[i][0] = src[cq];
      xa[i][1] = src[cq + 4];
    }
  };

  f32x4 acc[MW][NF];
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int st, const u32x4 (&xa)[MW][2]) {
#pragma unroll
    for (int p = 0; p < NPL; ++p)
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int r = p * Epad + f * 16 + l16;
        const u32x4 b0 = lds[st * STAGE + r * 8 + (cq ^ (r & 7))];
        const u32x4 b1 = lds[st * STAGE + r * 8 + ((cq + 4) ^ (r & 7))];
#pragma unroll
        for (int i = 0; i < MW; ++i) {
          acc[i][f] = mma16(xa[i][0], b0, acc[i][f], TW());
          acc[i][f] = mma16(xa[i][1], b1, acc[i][f], TW());
        }
      }
  };

  // two register sets for x, alternating; chunk c+1 is in flight during chunk c
  u32x4 xa0[MW][2], xa1[MW][2];
  if (c0 < c1) issue(c0, 0, xa0);
  for (int c = c0; c < c1; c += 2) {
    if (c + 1 < c1) { issue(c + 1, 1, xa1); wait_vmcnt<NL>(); } else { wait_vmcnt0(); }
    __syncthreads();
    compute(0, xa0);
    __syncthreads();
    if (c + 1 >= c1) break;
    if (c + 2 < c1) { issue(c + 2, 0, xa0); wait_vmcnt<NL>(); } else { wait_vmcnt0(); }
    __syncthreads();
    compute(1, xa1);
    __syncthreads();
  }
  // store partial scores: acc[i][f][v] = C[row 4*(lane/16)+v][col lane%16]
  float *out = part + (size_t)ks * T * E;
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      int e = f * 16 + l16;
      if (e >= Eh) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int t = tok0 + wv * 16 * MW + i * 16 + 4 * (lane >> 4) + v;
        if (t < T) out[(size_t)t * E + h * Eh + e] = acc[i][f][v];
      }
    }
}

// ------------------------------------------------------------------ selection
// L lanes (a power of two <= 16) per (token, head) pair; lane j of a pair owns
// local experts j, j+L, j+2L, ...  (at most EPL of them).
// sel_bias != NULL: selection (and group scores) on the float32 keys p + b
// instead of the scores; the gate is p, plus b when sel_gate.  all_experts:
// the token lists every expert of its head in index order with gate p (expert
// choice; no top-k).  probs != NULL: p of every expert is written out.
template <int EPL, int KMAX>
__global__ __launch_bounds__(256) void route_select_kernel(
    const float *__restrict__ part, int nsplit, const float *__restrict__ bias,
    float *__restrict__ logits_out, int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
    float *__restrict__ aux_p, int32_t *__restrict__ aux_c,
    int T, int H, int E, int Eh, int k, int L, int n_groups, int topk_groups, int renorm,
    const float *__restrict__ sel_bias, int sel_gate, int all_experts, float *__restrict__ probs) {
  extern __shared__ float sh[];  // [pairs_per_block][Eh] probabilities for the aux partials
  const int tid = threadIdx.x;
  const int ppb = 256 / L;
  const int pr = tid / L, j = tid % L;
  const long pair = (long)blockIdx.x * ppb + pr;
  const bool valid = pair < (long)T * H;
  const int t = valid ? (int)(pair / H) : 0;
  const int h = valid ? (int)(pair % H) : 0;
  const float NEG = -__builtin_huge_valf();

  float lv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = j + L * i;
    float v = NEG;
    if (valid && e < Eh) {
      size_t off = (size_t)t * E + h * Eh + e;
      v = part[off];
      for (int s = 1; s < nsplit; ++s) v += part[(size_t)s * T * E + off];
      if (bias) v += bias[h * Eh + e];
      v += 0.0f;  // -0.0 -> +0.0
      if (logits_out) logits_out[off] = v;
    }
    lv[i] = v;
  }
  // softmax statistics over the head's experts
  float m = NEG;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, lv[i]);
  m = wave_max(m, L);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s += (j + L * i < Eh) ? __expf(lv[i] - m) : 0.f;
  s = group_sum_fixed(s, L);
  if (probs && valid) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = j + L * i;
      if (e < Eh) probs[(size_t)t * E + h * Eh + e] = __expf(lv[i] - m) / s;
    }
  }
  if (all_experts) {  // expert choice: slot e = expert e, gate p (one head)
    if (valid) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = j + L * i;
        if (e < Eh) {
          topk_idx[(size_t)t * Eh + e] = e;
          topk_w[(size_t)t * Eh + e] = __expf(lv[i] - m) / s;
        }
      }
    }
    if (aux_p) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = j + L * i;
        if (e < Eh) sh[pr * Eh + e] = valid ? __expf(lv[i] - m) / s : 0.f;
      }
      __syncthreads();
      const long first = (long)blockIdx.x * ppb;
      const int nvalid = (int)min((long)ppb, (long)T * H - first);
      for (int e = tid; e < Eh; e += 256) {
        float acc = 0.f;
        for (int q = 0; q < ppb; ++q) acc += sh[q * Eh + e];
        aux_p[(size_t)blockIdx.x * Eh + e] = acc;
        atomicAdd(&aux_c[e], nvalid);  // every token offers every expert
      }
    }
    return;
  }
  // selection keys: the scores, or p + b under the balancing bias
  float kv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = j + L * i;
    kv[i] = lv[i];
    if (sel_bias && valid && e < Eh) kv[i] = (__expf(lv[i] - m) / s + sel_bias[h * Eh + e]) + 0.0f;
  }

  // group-limited: allowed-group bitmask (groups of consecutive experts)
  uint32_t allowed = 0xFFFFFFFFu;
  int grp[EPL];  // group of each owned expert (groups are consecutive experts)
  if (n_groups > 0) {
    // group score = largest score in the group; keep the topk_groups best
    // groups (higher score first, lower group index on ties)
    const int gsz = Eh / n_groups;
#pragma unroll
    for (int i = 0; i < EPL; ++i) grp[i] = (j + L * i) / gsz;
    uint32_t gkey[32];
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      float v = NEG;
      if (g < n_groups) {
#pragma unroll
        for (int i = 0; i < EPL; ++i)
          if (j + L * i < Eh && grp[i] == g) v = fmaxf(v, kv[i]);
        v = wave_max(v, L);
      }
      gkey[g] = score_key(v);
    }
    allowed = 0;
    for (int r = 0; r < topk_groups; ++r) {
      uint64_t best = 0;
#pragma unroll
      for (int g = 0; g < 32; ++g) {
        uint64_t c = ((uint64_t)gkey[g] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)g);
        if (g < n_groups && !((allowed >> g) & 1u) && c > best) best = c;
      }
      allowed |= 1u << (0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    }
  }
  // top-k: composite key (score key, inverted index) -> max = best, lower index on ties
  uint64_t kk[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = j + L * i;
    bool ok = e < Eh;
    if (ok && n_groups > 0) ok = (allowed >> grp[i]) & 1u;
    kk[i] = ok ? (((uint64_t)score_key(kv[i]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  int sel_e[KMAX];
  float sel_l[KMAX];
#pragma unroll
  for (int r = 0; r < KMAX; ++r) {
    if (r >= k) break;
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) best = kk[i] > best ? kk[i] : best;
    for (int o = L >> 1; o > 0; o >>= 1) {
      uint64_t other = __shfl_xor(best, o, WAVE);
      best = other > best ? other : best;
    }
    int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFull));
    float lb = NEG;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (kk[i] == best) { kk[i] = 0; }
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (j + L * i == e) lb = lv[i];
    lb = wave_max(lb, L);
    sel_e[r] = e;
    sel_l[r] = lb;
  }
  if (valid && j == 0) {
    float wsum = 0.f;
    float wr[KMAX];
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r >= k) break;
      wr[r] = __expf(sel_l[r] - m) / s;
      if (sel_bias && sel_gate) wr[r] += sel_bias[h * Eh + sel_e[r]];
      wsum += wr[r];
    }
#pragma unroll
    for (int r = 0; r < KMAX; ++r) {
      if (r >= k) break;
      size_t o = (size_t)t * H * k + h * k + r;
      topk_idx[o] = h * Eh + sel_e[r];
      topk_w[o] = renorm ? wr[r] / wsum : wr[r];
    }
  }
  if (aux_p) {  // H == 1: per-block column sums of p and choice counts
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = j + L * i;
      if (e < Eh) sh[pr * Eh + e] = valid ? __expf(lv[i] - m) / s : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < Eh; e += 256) {
      float acc = 0.f;
      for (int q = 0; q < ppb; ++q) acc += sh[q * Eh + e];
      aux_p[(size_t)blockIdx.x * Eh + e] = acc;
    }
    if (valid && j == 0)
      for (int r = 0; r < k; ++r) atomicAdd(&aux_c[sel_e[r]], 1);
  }
}

// aux = sum_e (sum_b aux_p[b][e] / T) * c_e / T, reduced in a fixed order
__global__ void route_aux_kernel(const float *__restrict__ aux_p, const int32_t *__restrict__ aux_c,
                                 int nblocks, int E, int T, float *__restrict__ aux) {
  __shared__ float red[256];
  float v = 0.f;
  for (int e = threadIdx.x; e < E; e += 256) {
    float me = 0.f;
    for (int b = 0; b < nblocks; ++b) me += aux_p[(size_t)b * E + e];
    v += (me / (float)T) * ((float)aux_c[e] / (float)T);
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

__global__ void zero_i32_kernel(int32_t *p, long n) {
  for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0;
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
  g.Epad = g.nf * 16;
  g.nplanes = (s.router_f32 && !s.act_f32) ? 3 : 1;
  int elem = s.act_f32 ? 4 : 2;
  int chunk = 128 / elem;
  int nchunks = s.dh / chunk;
  // token tile: 128 rows for wide routers (fewer re-reads of W_r), else 64
  g.mw = (g.nf >= 8) ? 2 : 1;
  g.tb = 64 * g.mw;
  long tiles = ((long)s.T + g.tb - 1) / g.tb * s.H;
  int ksplit = 1;
  while (tiles * ksplit < 256 && ksplit * 2 <= nchunks && ksplit < 8) ksplit *= 2;
  g.ksplit = ksplit;
  g.kchunk_per_split = (nchunks + ksplit - 1) / ksplit;
  g.L = 1;
  while (g.L < 16 && g.L * 16 < s.Eh) g.L *= 2;
  g.epl = (s.Eh + g.L - 1) / g.L;
  g.sel_blocks = (int)(((long)s.T * s.H + (256 / g.L) - 1) / (256 / g.L));
  return g;
}

size_t route_ws_bytes(const Shape &s) {
  RouteGeom g = route_geometry(s);
  size_t b = 0;
  b += align_up((size_t)g.ksplit * s.T * s.E * 4, 256);                  // partial scores
  if (g.nplanes == 3) b += align_up((size_t)s.H * 3 * g.Epad * s.dh * 2, 256);
  b += align_up((size_t)g.sel_blocks * s.Eh * 4, 256);                   // aux partials
  b += align_up((size_t)s.E * 4, 256);                                    // aux counts
  if (s.seq_len > 0) {
    const size_t nb = (size_t)(s.T / s.seq_len) * ((s.seq_len + SEQ_CH - 1) / SEQ_CH);
    b += align_up((size_t)s.T * s.E * 4, 256);                            // probabilities
    b += 2 * align_up(nb * s.E * 4, 256);                                  // chunk sums and counts
  }
  return b;
}

#define LAUNCH_CHECK() do { if (int rc_ = launch_status("route")) return rc_; } while (0)

template <typename TIN, typename TW, int NF, int NPL, int MW>
static void launch_logits(const Shape &s, const RouteGeom &g, const void *x, const void *w, float *part,
                          hipStream_t st) {
  dim3 grid((s.T + g.tb - 1) / g.tb, s.H, g.ksplit);
  // weights: direct [E][dh] (head stride E_h rows) or planes [H][3][Epad][dh]
  long head_stride = (NPL == 3) ? 3L * g.Epad * s.dh : (long)s.Eh * s.dh;
  long plane_stride = (long)g.Epad * s.dh;
  hipLaunchKernelGGL((route_logits_kernel<TIN, TW, NF, NPL, MW>), grid, dim3(256), 0, st,
                     (const TIN *)x, (const TW *)w, part, s.T, s.E, s.Eh, s.dh, s.H * s.dh,
                     g.kchunk_per_split, head_stride, plane_stride);
}

template <typename TIN, typename TW, int NPL>
static int dispatch_logits(const Shape &s, const RouteGeom &g, const void *x, const void *w, float *part,
                           hipStream_t st) {
  switch (g.nf) {
    case 1: launch_logits<TIN, TW, 1, NPL, 1>(s, g, x, w, part, st); break;
    case 2: launch_logits<TIN, TW, 2, NPL, 1>(s, g, x, w, part, st); break;
    case 3: launch_logits<TIN, TW, 3, NPL, 1>(s, g, x, w, part, st); break;
    case 4: launch_logits<TIN, TW, 4, NPL, 1>(s, g, x, w, part, st); break;
    case 5: launch_logits<TIN, TW, 5, NPL, 1>(s, g, x, w, part, st); break;
    case 6: launch_logits<TIN, TW, 6, NPL, 1>(s, g, x, w, part, st); break;
    default:
      if constexpr (NPL == 1) {
        switch (g.nf) {
          case 8: launch_logits<TIN, TW, 8, NPL, 2>(s, g, x, w, part, st); return 0;
          case 10: launch_logits<TIN, TW, 10, NPL, 2>(s, g, x, w, part, st); return 0;
          case 12: launch_logits<TIN, TW, 12, NPL, 2>(s, g, x, w, part, st); return 0;
          case 16: launch_logits<TIN, TW, 16, NPL, 2>(s, g, x, w, part, st); return 0;
        }
      }
      return -2;
  }
  return 0;
}

bool route_supported(const Shape &s) {
  RouteGeom g = route_geometry(s);
  // the three-plane (fp32 router, bf16 activations) form stages 3x the rows:
  // instantiated up to 6 fragments (E_h <= 96)
  if (g.nplanes == 3 && g.nf > 6) return false;
  return g.nf > 0 && g.epl <= 16;
}

int launch_route(const Shape &s, const void *x, const void *w_router, const float *bias, const float *sel_bias,
                 float *logits, int mode, int32_t *topk_idx, float *topk_w, float *aux_loss, float *seq_loss,
                 void *ws, hipStream_t st) {
  RouteGeom g = route_geometry(s);
  char *p = (char *)ws;
  float *part = (float *)p;
  p += align_up((size_t)g.ksplit * s.T * s.E * 4, 256);
  uint16_t *planes = nullptr;
  if (g.nplanes == 3) {
    planes = (uint16_t *)p;
    p += align_up((size_t)s.H * 3 * g.Epad * s.dh * 2, 256);
  }
  float *aux_p = (float *)p;
  p += align_up((size_t)g.sel_blocks * s.Eh * 4, 256);
  int32_t *aux_c = (int32_t *)p;
  p += align_up((size_t)s.E * 4, 256);
  float *probs = nullptr, *psum = nullptr;
  int32_t *pcnt = nullptr;
  const int nseq = s.seq_len > 0 ? s.T / s.seq_len : 0, nch = s.seq_len > 0 ? (s.seq_len + SEQ_CH - 1) / SEQ_CH : 0;
  if (seq_loss) {
    probs = (float *)p;
    p += align_up((size_t)s.T * s.E * 4, 256);
    psum = (float *)p;
    p += align_up((size_t)nseq * nch * s.E * 4, 256);
    pcnt = (int32_t *)p;
  }

  const float *src = part;
  int nsplit = g.ksplit;
  if (mode == 2) {  // LOAD
    src = logits;
    nsplit = 1;
    bias = nullptr;
  } else {
    int rc;
    if (s.act_f32) {
      // f32 activations with an f32 router: f32 MFMA
      rc = dispatch_logits<float, float, 1>(s, g, x, w_router, part, st);
    } else if (g.nplanes == 3) {
      int n = s.H * g.Epad * s.dh;
      hipLaunchKernelGGL(route_split_w_kernel, dim3(min(1024, (n + 255) / 256)), dim3(256), 0, st,
                         (const float *)w_router, planes, s.E, g.Epad, s.dh, s.H, s.Eh);
      LAUNCH_CHECK();
      rc = dispatch_logits<uint16_t, uint16_t, 3>(s, g, x, planes, part, st);
    } else {
      rc = dispatch_logits<uint16_t, uint16_t, 1>(s, g, x, w_router, part, st);
    }
    if (rc) return rc;
    LAUNCH_CHECK();
  }
  float *lout = (mode == 1) ? logits : nullptr;
  bool aux = aux_loss != nullptr;
  if (aux) {
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(256), 0, st, aux_c, (long)s.E);
    LAUNCH_CHECK();
  }
  size_t shm = aux ? (size_t)(256 / g.L) * s.Eh * 4 : 0;
#define SEL(EPL_)                                                                                   \
  hipLaunchKernelGGL((route_select_kernel<EPL_, 8>), dim3(g.sel_blocks), dim3(256), shm, st, src, nsplit, \
                     bias, lout, topk_idx, topk_w, aux ? aux_p : nullptr, aux_c, s.T, s.H, s.E, s.Eh, s.k,   \
                     g.L, s.n_groups, s.topk_groups, s.renorm, s.expert_choice ? nullptr : sel_bias, s.sel_gate, \
                     s.expert_choice, probs)
  if (g.epl <= 4) SEL(4);
  else if (g.epl <= 8) SEL(8);
  else SEL(16);
#undef SEL
  LAUNCH_CHECK();
  if (aux) {
    hipLaunchKernelGGL(route_aux_kernel, dim3(1), dim3(256), 0, st, aux_p, aux_c, g.sel_blocks, s.E, s.T,
                       aux_loss);
    LAUNCH_CHECK();
  }
  if (seq_loss) {
    hipLaunchKernelGGL(route_seq_part_kernel, dim3((unsigned)(nseq * nch)), dim3(256), (size_t)s.E * 4, st, probs,
                       topk_idx, s.E, s.K, s.seq_len, nch, psum, pcnt);
    LAUNCH_CHECK();
    hipLaunchKernelGGL(route_seq_kernel, dim3((unsigned)nseq), dim3(256), 0, st, psum, pcnt, s.E, s.seq_len, nch,
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
