// C-ABI entry points of libmoe.so (declared and documented in include/moe.h).
// Host code only: validation, workspace layout and launch order.  Every check
// runs before the first launch, so a rejected call launches nothing.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/moe.h"
#include "launch.h"

using moe::Shape;

int moe::launch_status(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return 0;
  if (getenv("MOE_DEBUG")) fprintf(stderr, "moe: %s launch failed: %s\n", what, hipGetErrorString(e));
  return -4;
}

namespace {

size_t al(size_t v) { return (v + 255) / 256 * 256; }

// config -> Shape; returns a moe_status
int make_shape(const moe_config *c, Shape *s) {
  if (!c) return MOE_ERR_ARG;
  if (c->T < 0 || c->d_model <= 0 || c->d_model % 64 || c->n_heads < 1 || c->d_head <= 0 || c->d_head % 64)
    return MOE_ERR_ARG;
  if (!c->latent_proj && (long)c->n_heads * c->d_head != c->d_model) return MOE_ERR_ARG;
  if (c->n_experts < 1 || c->n_experts % c->n_heads) return MOE_ERR_ARG;
  const int Eh = c->n_experts / c->n_heads;
  if (c->top_k < 1 || c->top_k > Eh) return MOE_ERR_ARG;
  if (c->n_groups < 0) return MOE_ERR_ARG;
  if (c->n_groups > 0) {
    if (Eh % c->n_groups || c->topk_groups < 1 || c->topk_groups > c->n_groups) return MOE_ERR_ARG;
    if ((long)c->top_k > (long)c->topk_groups * (Eh / c->n_groups)) return MOE_ERR_ARG;
  }
  if ((c->renorm != 0 && c->renorm != 1) || c->drop < 0 || c->drop > 2) return MOE_ERR_ARG;
  if (c->drop == MOE_DROP_CAPACITY && c->capacity < 0) return MOE_ERR_ARG;
  if (c->drop == MOE_DROP_AFFINITY && (c->keep_num <= 0 || c->keep_den <= 0 || c->keep_num > c->keep_den))
    return MOE_ERR_ARG;
  if (c->d_ff <= 0 || c->d_ff % 64 || (c->act != MOE_ACT_RELU && c->act != MOE_ACT_SWIGLU)) return MOE_ERR_ARG;
  if (c->n_shared < 0 || (c->latent_proj != 0 && c->latent_proj != 1) || (c->residual != 0 && c->residual != 1))
    return MOE_ERR_ARG;
  if ((c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) ||
      (c->router_dtype != MOE_F32 && c->router_dtype != MOE_BF16))
    return MOE_ERR_ARG;
  // supported subset
  if (c->top_k > 8 || Eh > 256 || c->n_experts > 1024 || c->n_groups > 32) return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_F32 && c->router_dtype == MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->n_shared > 0 && (c->n_heads != 1 || c->latent_proj)) return MOE_ERR_UNSUPPORTED;
  if ((long)c->T * c->n_heads * c->top_k > 0x7FFFFFFFL) return MOE_ERR_UNSUPPORTED;
  s->T = c->T; s->d = c->d_model; s->H = c->n_heads; s->dh = c->d_head; s->E = c->n_experts; s->Eh = Eh;
  s->k = c->top_k; s->K = c->n_heads * c->top_k;
  s->n_groups = c->n_groups; s->topk_groups = c->topk_groups; s->renorm = c->renorm;
  s->drop = c->drop; s->C = c->capacity; s->keep_num = c->keep_num; s->keep_den = c->keep_den;
  s->dff = c->d_ff; s->act = c->act; s->n_shared = c->n_shared; s->latent = c->latent_proj;
  s->residual = c->residual;
  s->act_f32 = c->act_dtype == MOE_F32;
  s->router_f32 = c->router_dtype == MOE_F32;
  long tk = (long)s->T * s->K;
  s->R_max = (s->drop == MOE_DROP_CAPACITY) ? (tk < (long)s->E * s->C ? tk : (long)s->E * s->C) : tk;
  if (!moe::route_supported(*s)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t scratch_bytes(const Shape &s) {
  size_t m = moe::route_ws_bytes(s);
  size_t v = moe::dispatch_ws_bytes(s);
  if (v > m) m = v;
  v = moe::ffn_ws_bytes(s);
  if (v > m) m = v;
  v = moe::dense_ws_bytes();
  if (v > m) m = v;
  return m;
}

// intermediates of moe_layer_fwd, in workspace order
struct LayerBufs {
  size_t topk_idx, topk_w, demand, counts, offsets, row_of, src_of, aux, z, y_perm, shared, o, scratch, total;
};

LayerBufs layer_layout(const Shape &s) {
  const size_t esz = s.act_f32 ? 4 : 2;
  const size_t tk = (size_t)s.T * s.K;
  LayerBufs b{};
  size_t o = 0;
  b.topk_idx = o; o += al(tk * 4);
  b.topk_w = o; o += al(tk * 4);
  b.demand = o; o += al((size_t)s.E * 4);
  b.counts = o; o += al((size_t)s.E * 4);
  b.offsets = o; o += al((size_t)(s.E + 1) * 4);
  b.row_of = o; o += al(tk * 4);
  b.src_of = o; o += al((size_t)s.R_max * 4);
  b.aux = o; o += al(4);
  b.z = o; o += s.latent ? al((size_t)s.T * s.H * s.dh * esz) : 0;
  b.y_perm = o; o += al((size_t)s.R_max * s.dh * esz);
  b.shared = o; o += s.n_shared ? al((size_t)s.T * s.d * esz) : 0;
  b.o = o; o += s.latent ? al((size_t)s.T * s.H * s.dh * esz) : 0;
  b.scratch = o; o += scratch_bytes(s);
  b.total = o;
  return b;
}

int check_ws(const Shape &s, const void *ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return MOE_ERR_WORKSPACE;
  if (ws_bytes < layer_layout(s).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// HIP's last-error state also holds errors of earlier, unrelated runtime
// calls of the caller; clear it before our first launch so that the checks
// after each launch see only our own launches
void clear_stale_error() { (void)hipGetLastError(); }

// the gathered operand rows are addressed with 32-bit element offsets into x
bool gather_supported(const Shape &s) { return (long)s.T * s.H * s.dh < (1L << 31); }

int rc_of(int launcher_rc) {
  if (launcher_rc == -2) return MOE_ERR_UNSUPPORTED;
  if (launcher_rc != 0) return MOE_ERR_HIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config *cfg) {
  Shape s;
  if (make_shape(cfg, &s) != MOE_OK) return 0;
  return layer_layout(s).total;
}

int64_t moe_rows_upper_bound(const moe_config *cfg) {
  Shape s;
  if (make_shape(cfg, &s) != MOE_OK) return -1;
  return s.R_max;
}

const char *moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid request outside the supported shapes";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small or not 256-byte aligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    default: return "unknown moe_status";
  }
}

int moe_check_config(const moe_config *cfg) {
  Shape s;
  return make_shape(cfg, &s);
}

int moe_route(const moe_config *cfg, const void *x, const void *w_router, const float *bias, float *logits,
              int mode, int32_t *topk_idx, float *topk_w, float *aux_loss, void *ws, size_t ws_bytes,
              hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (mode < MOE_LOGITS_COMPUTE || mode > MOE_LOGITS_LOAD) return MOE_ERR_ARG;
  if (!topk_idx || !topk_w) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_LOAD && (!x || !w_router)) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_COMPUTE && !logits) return MOE_ERR_ARG;
  if (aux_loss && s.H != 1) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_route(s, x, w_router, bias, logits, mode, topk_idx, topk_w, aux_loss, ws, stream));
}

int moe_dispatch(const moe_config *cfg, const int32_t *topk_idx, const float *topk_w, const void *x,
                 int32_t *demand, int32_t *counts, int32_t *offsets, int32_t *row_of, int32_t *src_of, void *x_perm,
                 void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!topk_idx || !demand || !counts || !offsets || !row_of || (!src_of && s.R_max) || (x_perm && !x))
    return MOE_ERR_ARG;
  if (s.drop == MOE_DROP_AFFINITY && !topk_w) return MOE_ERR_ARG;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_dispatch(s, topk_idx, topk_w, x, demand, counts, offsets, row_of, src_of, x_perm, ws,
                                    stream));
}

int moe_expert_ffn(const moe_config *cfg, const void *x_perm, const int32_t *offsets, const void *w1, const void *w3,
                   const void *w2, void *y_perm, const void *x_shared, const void *ws1, const void *ws3,
                   const void *ws2, void *shared_out, void *ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (((!x_perm || !y_perm) && s.R_max) || !offsets || !w1 || !w2) return MOE_ERR_ARG;
  if ((s.act == MOE_ACT_SWIGLU) != (w3 != nullptr)) return MOE_ERR_ARG;
  if (s.n_shared) {
    if (!x_shared || !ws1 || !ws2 || !shared_out) return MOE_ERR_ARG;
    if ((s.act == MOE_ACT_SWIGLU) != (ws3 != nullptr)) return MOE_ERR_ARG;
  }
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_expert_ffn(s, x_perm, nullptr, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2,
                                      shared_out, ws, stream));
}

int moe_expert_ffn_gather(const moe_config *cfg, const void *x, const int32_t *src_of, const int32_t *offsets,
                          const void *w1, const void *w3, const void *w2, void *y_perm, const void *x_shared,
                          const void *ws1, const void *ws3, const void *ws2, void *shared_out, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (((!x || !src_of || !y_perm) && s.R_max) || !offsets || !w1 || !w2) return MOE_ERR_ARG;
  if ((s.act == MOE_ACT_SWIGLU) != (w3 != nullptr)) return MOE_ERR_ARG;
  if (s.n_shared) {
    if (!x_shared || !ws1 || !ws2 || !shared_out) return MOE_ERR_ARG;
    if ((s.act == MOE_ACT_SWIGLU) != (ws3 != nullptr)) return MOE_ERR_ARG;
  }
  if (!gather_supported(s)) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_expert_ffn(s, x, src_of, offsets, w1, w3, w2, y_perm, x_shared, ws1, ws3, ws2,
                                      shared_out, ws, stream));
}

int moe_combine(const moe_config *cfg, const void *y_perm, const int32_t *row_of, const float *topk_w,
                const void *residual, const void *shared_out, void *y, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  if (!y_perm || !row_of || !topk_w || !y) return MOE_ERR_ARG;
  if (s.T == 0) return MOE_OK;
  clear_stale_error();
  return rc_of(moe::launch_combine(s, y_perm, row_of, topk_w, residual, shared_out, y, stream));
}

int moe_layer_fwd(const moe_config *cfg, const moe_weights *w, const void *x, void *y, moe_layer_io *io, void *ws,
                  size_t ws_bytes, hipStream_t stream) {
  Shape s;
  int rc = make_shape(cfg, &s);
  if (rc) return rc;
  moe_layer_io none;
  memset(&none, 0, sizeof(none));
  if (!io) io = &none;
  const int mode = io->logits_mode;
  if (!w || !x || !y || x == y) return MOE_ERR_ARG;
  if (mode < MOE_LOGITS_COMPUTE || mode > MOE_LOGITS_LOAD) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_COMPUTE && !io->logits) return MOE_ERR_ARG;
  if (mode != MOE_LOGITS_LOAD && !w->w_router) return MOE_ERR_ARG;
  if (!w->w1 || !w->w2 || ((s.act == MOE_ACT_SWIGLU) != (w->w3 != nullptr))) return MOE_ERR_ARG;
  if (s.n_shared && (!w->ws1 || !w->ws2 || ((s.act == MOE_ACT_SWIGLU) != (w->ws3 != nullptr)))) return MOE_ERR_ARG;
  if (s.latent && (!w->w_in || !w->w_out)) return MOE_ERR_ARG;
  if (io->aux_loss && s.H != 1) return MOE_ERR_UNSUPPORTED;
  if (!io->x_perm && !gather_supported(s)) return MOE_ERR_UNSUPPORTED;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (s.T == 0) return MOE_OK;

  const LayerBufs L = layer_layout(s);
  char *base = (char *)ws;
  auto pick = [&](void *user, size_t off) -> void * { return user ? user : (void *)(base + off); };
  int32_t *topk_idx = (int32_t *)pick(io->topk_idx, L.topk_idx);
  float *topk_w = (float *)pick(io->topk_w, L.topk_w);
  int32_t *demand = (int32_t *)pick(io->demand, L.demand);
  int32_t *counts = (int32_t *)pick(io->counts, L.counts);
  int32_t *offsets = (int32_t *)pick(io->offsets, L.offsets);
  int32_t *row_of = (int32_t *)pick(io->row_of, L.row_of);
  int32_t *src_of = (int32_t *)pick(io->src_of, L.src_of);
  void *x_perm = io->x_perm;  // NULL: the expert FFN gathers rows from xin
  void *y_perm = pick(io->y_perm, L.y_perm);
  void *shared = s.n_shared ? pick(io->shared_out, L.shared) : nullptr;
  void *z = s.latent ? pick(io->z, L.z) : nullptr;
  void *o = s.latent ? pick(io->o, L.o) : nullptr;
  void *scratch = base + L.scratch;

  clear_stale_error();
  const void *xin = x;  // router and expert input
  if (s.latent) {
    if ((rc = rc_of(moe::launch_dense(s.act_f32, x, w->w_in, z, nullptr, s.T, s.H * s.dh, s.d, scratch, stream))))
      return rc;
    xin = z;
  }
  if ((rc = rc_of(moe::launch_route(s, xin, w->w_router, w->router_bias, io->logits, mode, topk_idx, topk_w,
                                    io->aux_loss, scratch, stream))))
    return rc;
  if ((rc = rc_of(moe::launch_dispatch(s, topk_idx, topk_w, xin, demand, counts, offsets, row_of, src_of, x_perm,
                                       scratch, stream))))
    return rc;
  if ((rc = rc_of(moe::launch_expert_ffn(s, x_perm ? x_perm : xin, x_perm ? nullptr : src_of, offsets, w->w1,
                                         w->w3, w->w2, y_perm, x, w->ws1, w->ws3, w->ws2, shared, scratch,
                                         stream))))
    return rc;
  const void *res = (!s.latent && s.residual) ? x : nullptr;
  if ((rc = rc_of(moe::launch_combine(s, y_perm, row_of, topk_w, res, shared, s.latent ? o : y, stream))))
    return rc;
  if (s.latent) {
    if ((rc = rc_of(moe::launch_dense(s.act_f32, o, w->w_out, y, x, s.T, s.d, s.H * s.dh, scratch, stream))))
      return rc;
  }
  return MOE_OK;
}

}  // extern "C"
