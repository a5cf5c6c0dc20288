// C ABI of libawq (declared in include/awq.h): argument validation, workspace
// carving and kernel launches.  Every argument error is found before anything
// is enqueued; no entry point allocates device memory.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/awq.h"
#include "awq_device.h"
#include "awq_launch.h"

using namespace awq;

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

// records the timing events, if set, on `stream`
void mark(bool before, hipStream_t stream) {
  hipEvent_t e = before ? g_ev_before : g_ev_after;
  if (e != nullptr) (void)hipEventRecord(e, stream);
}

awq_status fail(awq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

awq_status ok() {
  g_err[0] = '\0';
  return AWQ_OK;
}

awq_status hip_status(hipError_t e, const char* where) {
  if (e != hipSuccess) return fail(AWQ_EHIP, "%s: %s", where, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

bool valid_group(int32_t g) { return g == 32 || g == 64 || g == 128; }

// workspace layout of awq_search_scales
struct SearchPlan {
  bool output;
  int64_t n_blocks;     // weight score: search blocks
  int64_t T_pad, d_out_pad, K_pad, n_mt, ldc;  // output score: padded GEMM shapes, token tiles, partial ld
  int64_t n_x, n_db;    // output score: X max partials, dW bounds per candidate (1)
  int cand_chunk;       // output score: candidates per dW chunk
  bool gram;            // alpha search in the second-moment form (H = X^T X)
  bool clip_gram;       // clip search in the second-moment form (only when forced)
  bool need_x16, need_h;  // operands of the direct form / of the second-moment form
  int64_t n_mt_a, n_mt_c;  // rows of column partials: alpha search, clip search
  int64_t g_T_pad, g_xt_rows, g_h_rows;  // second-moment form: token padding, Xt rows, H16 rows
  size_t off_S, off_C2, off_tot, off_part, off_x16, off_xt, off_dw, off_xmax, off_dmax, off_sc, off_chunk, total;
  size_t off_h32, off_h16, off_hc, off_hr, off_cpart, off_cmax;
  bool duo;                   // duo-scaling candidates: w_mean, its scratch, the fp64 table
  size_t off_wmean, off_rmax, off_wpart, off_T, off_ext;
};

// scratch of the duo candidates, from `off` on
size_t plan_duo(SearchPlan& p, int64_t d_out, int64_t d_in, int n_grid, size_t off) {
  p.off_wmean = off;
  off += align256((size_t)d_in * sizeof(float));
  p.off_rmax = off;
  off += align256((size_t)d_out * sizeof(float));
  p.off_wpart = off;
  off += align256((size_t)wmean_splits(d_out) * d_in * sizeof(double));
  p.off_T = off;
  off += align256((size_t)n_grid * d_in * sizeof(double));
  p.off_ext = off;
  off += align256((size_t)n_grid * duo_cand_blocks(d_in) * 2 * sizeof(double));
  return off;
}

constexpr size_t kDwBudget = (size_t)2 << 30;  // bytes of dW per chunk (2 GiB)

// Alpha search of the output score in the second-moment form?  Forced by a
// flag, else taken when its matrix-core work (H = X^T X once, then d_in^2 per
// scored row) is below 0.8 of the direct form's (T d_in per scored row); the
// margin covers its extra passes (transpose of X, H to fp16).  The clip search
// decides per row, and the error of one row's quadratic form over an fp16 H''
// grows with the conditioning of X^T X (linearly; the direct form's with its
// square root), where the alpha search's sums over rows are carried by the
// well-measured rows: in the second-moment form the clip search takes H'' as
// hi + lo parts (use_gram_clip).
// Its fp32 H and fp16 operands are addressed with 32-bit offsets.
bool gram_fits(const SearchPlan& p) {
  const double k = (double)p.K_pad;
  return k * k < 2147483648.0 && (double)p.g_h_rows * k * 4.0 < 4294967296.0 &&
         (double)p.g_xt_rows * (double)p.g_T_pad * 2.0 < 4294967296.0;
}

// Matrix-core work (multiply-adds) of the second-moment form for `rows` scored
// rows: H's tiles on and right of the diagonal blocks (once per search, when
// `with_h`), then K from each row tile's diagonal block on, `parts` times
// (1: H'' in fp16; 2: hi + lo)
double gram_work(const SearchPlan& p, double rows, int parts, bool with_h) {
  const int64_t bm = gemm_sq_tile_rows(), bn = 256;
  double h_tiles = 0.0, k_cols = 0.0;
  for (int64_t m0 = 0; m0 < p.g_h_rows; m0 += bm) {
    for (int64_t n0 = 0; n0 < p.K_pad; n0 += bn) h_tiles += (n0 + bn > m0) ? 1.0 : 0.0;
    k_cols += (double)(p.K_pad - m0);
  }
  return (with_h ? h_tiles * (double)(bm * bn) * (double)p.g_T_pad : 0.0) + parts * (double)bm * k_cols * rows;
}

bool use_gram(const awq_search_cfg& cfg, const SearchPlan& p, int64_t T) {
  (void)T;
  if (cfg.flags & AWQ_FLAG_OUT_DIRECT) return false;
  if (cfg.flags & AWQ_FLAG_OUT_GRAM) return true;
  if (!gram_fits(p)) return false;
  const double rows = (double)cfg.n_grid * (double)p.d_out_pad;
  return gram_work(p, rows, 1, true) < 0.8 * (double)p.T_pad * (double)p.K_pad * rows;
}

// The clip search in the second-moment form takes H'' as hi + lo (twice the
// products of the alpha search's form): taken when that is below 0.85 of the
// direct form's work (the split product, with twice the K per block, runs at
// the direct GEMM's fraction of the matrix-core peak: 0.47 of it on MLP
// gate/up and down), H counted only if the alpha search did not form it.
bool use_gram_clip(const awq_search_cfg& cfg, const SearchPlan& p) {
  if (cfg.n_clip < 2 || (cfg.flags & AWQ_FLAG_OUT_DIRECT)) return false;
  if (cfg.flags & AWQ_FLAG_OUT_GRAM) return true;
  if (!gram_fits(p)) return false;
  const double rows = (double)cfg.n_clip * (double)p.d_out_pad;
  return gram_work(p, rows, 2, !p.gram) < 0.85 * (double)p.T_pad * (double)p.K_pad * rows;
}

SearchPlan plan_search(const awq_search_cfg& cfg, int64_t d_out, int64_t d_in, int64_t T) {
  SearchPlan p{};
  p.output = cfg.score == AWQ_SCORE_OUTPUT;
  size_t off = 0;
  p.off_S = off;
  off += align256((size_t)cfg.n_grid * d_in * sizeof(float));
  p.off_tot = off;
  off += align256((size_t)kMaxGrid * sizeof(double));
  if (!p.output) {
    p.off_C2 = off;
    off += align256((size_t)cfg.n_grid * d_in * sizeof(float));
    p.n_blocks = search_weight_blocks(cfg.group_size, d_out, d_in);
    p.off_part = off;
    off += align256((size_t)p.n_blocks * cfg.n_grid * sizeof(float));
  } else {
    gemm_sq_pad(T, d_out, d_in, &p.T_pad, &p.d_out_pad, &p.K_pad);
    gram_pad(T, p.K_pad, &p.g_T_pad, &p.g_xt_rows, &p.g_h_rows);
    p.gram = use_gram(cfg, p, T);
    p.clip_gram = use_gram_clip(cfg, p);
    p.need_x16 = !p.gram || (cfg.n_clip >= 2 && !p.clip_gram);
    p.need_h = p.gram || p.clip_gram;
    p.n_mt_a = p.gram ? gram_units(p.g_h_rows) : p.T_pad / gemm_sq_tile_rows();
    p.n_mt_c = p.clip_gram ? gram_units(p.g_h_rows) : p.T_pad / gemm_sq_tile_rows();
    p.n_mt = cfg.n_clip >= 2 && p.n_mt_c > p.n_mt_a ? p.n_mt_c : p.n_mt_a;  // rows of column partials
    p.n_x = absmax_blocks(T);
    p.n_db = 1;  // one bound on max |dW| per candidate
    const int max_c = cfg.n_grid > cfg.n_clip ? cfg.n_grid : cfg.n_clip;
    p.ldc = (int64_t)max_c * p.d_out_pad;
    const size_t per_cand = (size_t)p.d_out_pad * p.K_pad * sizeof(uint16_t);
    int64_t chunk = (int64_t)(kDwBudget / per_cand);
    if (chunk > max_c) chunk = max_c;
    if (chunk < 1) chunk = 1;
    p.cand_chunk = (int)chunk;
    p.off_x16 = off;  // X16 [T_pad, K_pad] (direct form)
    if (p.need_x16) off += align256((size_t)p.T_pad * p.K_pad * sizeof(uint16_t));
    p.off_xt = off;   // Xt [g_xt_rows, g_T_pad] (second-moment form)
    if (p.need_h) off += align256((size_t)p.g_xt_rows * p.g_T_pad * sizeof(uint16_t));
    if (p.need_h) {
      int ns;
      int64_t slice;
      gram_slices(p.g_T_pad, p.K_pad, &ns, &slice);
      p.off_h32 = off;
      off += align256((size_t)ns * p.K_pad * p.K_pad * sizeof(float));
      p.off_h16 = off;  // hi and lo parts
      off += align256((size_t)p.g_h_rows * 2 * p.K_pad * sizeof(uint16_t));
      p.off_hc = off;
      off += align256((size_t)p.K_pad * sizeof(float));
      p.off_hr = off;
      off += align256((size_t)p.K_pad * sizeof(float));
    }
    p.off_dw = off;
    off += align256(per_cand * chunk);
    p.off_part = off;
    off += align256((size_t)p.n_mt * p.ldc * sizeof(float));
    p.off_xmax = off;
    off += align256((size_t)p.n_x * sizeof(float));
    p.off_dmax = off;
    off += align256((size_t)max_c * p.n_db * sizeof(float));
    p.off_sc = off;
    off += 2 * align256(sizeof(OutScales));
    p.off_chunk = off;
    off += align256((size_t)max_c * reduce_cols_chunks(d_out) * sizeof(double));
    p.off_cpart = off;
    off += align256((size_t)colmax_part_floats(d_in) * sizeof(float));
    p.off_cmax = off;
    off += align256((size_t)d_in * sizeof(float));
  }
  p.duo = (cfg.flags & AWQ_FLAG_DUO) != 0;
  if (p.duo) off = plan_duo(p, d_out, d_in, cfg.n_grid, off);
  p.total = off;
  return p;
}

// the candidate table of a search: plain, or duo scaling over the group's rows
hipError_t launch_cands(const awq_search_cfg& cfg, const SearchPlan& plan, const WParts& parts, int64_t d_out,
                        int64_t d_in, const float* x_mean, char* base, float* S, float* C2, hipStream_t s) {
  if (!plan.duo) return launch_candidates(x_mean, d_in, cfg.n_grid, cfg.s_min, S, C2, s);
  float* w_mean = (float*)(base + plan.off_wmean);
  hipError_t e = launch_weight_channel_mean(parts, d_out, d_in, (float*)(base + plan.off_rmax),
                                            (double*)(base + plan.off_wpart), w_mean, s);
  if (e != hipSuccess) return e;
  return launch_candidates_duo(x_mean, w_mean, d_in, cfg.n_grid, cfg.s_min, (double*)(base + plan.off_T),
                               (double*)(base + plan.off_ext), S, C2, s);
}

awq_status check_cfg(const awq_search_cfg* cfg) {
  if (!cfg) return fail(AWQ_EINVAL, "cfg is NULL");
  if (!valid_group(cfg->group_size)) return fail(AWQ_EINVAL, "group_size %d not in {32,64,128}", cfg->group_size);
  if (cfg->n_grid < 1 || cfg->n_grid > kMaxGrid) return fail(AWQ_EINVAL, "n_grid %d not in [1,%d]", cfg->n_grid, kMaxGrid);
  if (cfg->score != AWQ_SCORE_WEIGHT && cfg->score != AWQ_SCORE_OUTPUT)
    return fail(AWQ_EINVAL, "score %d unknown", cfg->score);
  if (cfg->n_clip != 0) {
    if (cfg->n_clip < 2 || cfg->n_clip > kMaxGrid) return fail(AWQ_EINVAL, "n_clip %d not 0 or in [2,%d]", cfg->n_clip, kMaxGrid);
    if (cfg->score != AWQ_SCORE_OUTPUT) return fail(AWQ_EINVAL, "clip search needs the output score");
    if (!(cfg->clip_lo > 0.0f && cfg->clip_lo <= 1.0f)) return fail(AWQ_EINVAL, "clip_lo %g not in (0,1]", (double)cfg->clip_lo);
  }
  if (!(cfg->s_min > 0.0 && isfinite(cfg->s_min))) return fail(AWQ_EINVAL, "s_min must be positive and finite");
  if (cfg->flags & ~(AWQ_FLAG_DUO | AWQ_FLAG_ASYM | AWQ_FLAG_OUT_DIRECT | AWQ_FLAG_OUT_GRAM))
    return fail(AWQ_EINVAL, "flags 0x%x: unknown bits", (unsigned)cfg->flags);
  if ((cfg->flags & AWQ_FLAG_OUT_DIRECT) && (cfg->flags & AWQ_FLAG_OUT_GRAM))
    return fail(AWQ_EINVAL, "AWQ_FLAG_OUT_DIRECT and AWQ_FLAG_OUT_GRAM exclude each other");
  return AWQ_OK;
}

}  // namespace

extern "C" {

const char* awq_last_error(void) { return g_err; }

awq_status awq_set_timing_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr)) return fail(AWQ_EINVAL, "set both events or neither");
  g_ev_before = (hipEvent_t)before;
  g_ev_after = (hipEvent_t)after;
  return ok();
}

int32_t awq_abi_version(void) { return AWQ_ABI_VERSION; }

// ---------------------------------------------------------------------------
awq_status awq_act_stats_workspace(int64_t T, int64_t d_in, size_t* bytes) {
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (T < 0 || d_in < 1) return fail(AWQ_EINVAL, "need T >= 0 and d_in >= 1");
  int64_t ns, rps;
  act_stats_plan(T, d_in, &ns, &rps);
  *bytes = align256((size_t)ns * d_in * sizeof(double));
  return ok();
}

awq_status awq_act_stats(const void* X, int32_t x_dtype, int64_t T, int64_t d_in, int64_t ld_x,
                         float inv_count, int32_t accumulate, float* x_mean, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  if (x_dtype != AWQ_F16 && x_dtype != AWQ_BF16) return fail(AWQ_EDTYPE, "x_dtype %d: need AWQ_F16 or AWQ_BF16", x_dtype);
  if (T < 0 || d_in < 1) return fail(AWQ_EINVAL, "need T >= 0 and d_in >= 1");
  if (ld_x < d_in) return fail(AWQ_ESHAPE, "ld_x %lld < d_in %lld", (long long)ld_x, (long long)d_in);
  if (!x_mean) return fail(AWQ_EINVAL, "x_mean is NULL");
  if (T > 0 && !X) return fail(AWQ_EINVAL, "X is NULL");
  if (!isfinite(inv_count)) return fail(AWQ_EINVAL, "inv_count not finite");
  size_t need = 0;
  awq_act_stats_workspace(T, d_in, &need);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(AWQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if (need > 0 && ((uintptr_t)ws & 7u)) return fail(AWQ_EALIGN, "ws not 8-byte aligned");
  mark(true, (hipStream_t)stream);
  hipError_t e = launch_act_stats(X, x_dtype == AWQ_BF16, T, d_in, ld_x, inv_count, accumulate ? 1 : 0, x_mean,
                                  ws, (hipStream_t)stream);
  mark(false, (hipStream_t)stream);
  return hip_status(e, "awq_act_stats");
}

// ---------------------------------------------------------------------------
awq_status awq_candidate_scales_workspace(int64_t d_in, int32_t n_grid, size_t* bytes) {
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (d_in < 1) return fail(AWQ_EINVAL, "d_in must be >= 1");
  if (n_grid < 1 || n_grid > kMaxGrid) return fail(AWQ_EINVAL, "n_grid %d not in [1,%d]", n_grid, kMaxGrid);
  *bytes = 0;  // the table needs no scratch
  return ok();
}

awq_status awq_candidate_scales(const float* x_mean, int64_t d_in, int32_t n_grid, double s_min,
                                float* S, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x_mean || !S) return fail(AWQ_EINVAL, "x_mean / S is NULL");
  if (d_in < 1) return fail(AWQ_EINVAL, "d_in must be >= 1");
  if (n_grid < 1 || n_grid > kMaxGrid) return fail(AWQ_EINVAL, "n_grid %d not in [1,%d]", n_grid, kMaxGrid);
  if (!(s_min > 0.0 && isfinite(s_min))) return fail(AWQ_EINVAL, "s_min must be positive and finite");
  (void)ws;
  (void)ws_bytes;
  return hip_status(launch_candidates(x_mean, d_in, n_grid, s_min, S, nullptr, (hipStream_t)stream),
                    "awq_candidate_scales");
}

// ---------------------------------------------------------------------------
// group parts of an awq_wgroup (validated), d_out in *d_out
static awq_status read_group(const awq_wgroup* W, WParts* parts, int64_t* d_out) {
  if (!W || !W->w || !W->rows) return fail(AWQ_EINVAL, "weight group is NULL");
  if (W->n_parts < 1 || W->n_parts > kMaxParts) return fail(AWQ_EINVAL, "n_parts %d not in [1,%d]", W->n_parts, kMaxParts);
  *parts = WParts{};
  parts->n = W->n_parts;
  int64_t n = 0;
  for (int p = 0; p < W->n_parts; ++p) {
    if (W->rows[p] < 0) return fail(AWQ_EINVAL, "rows[%d] < 0", p);
    if (W->rows[p] > 0 && !W->w[p]) return fail(AWQ_EINVAL, "w[%d] is NULL", p);
    if (!aligned16(W->w[p])) return fail(AWQ_EALIGN, "w[%d] not 16-byte aligned", p);
    parts->ptr[p] = (const uint16_t*)W->w[p];
    parts->row_start[p] = n;
    n += W->rows[p];
  }
  for (int p = W->n_parts; p <= kMaxParts; ++p) parts->row_start[p] = n;
  for (int p = W->n_parts; p < kMaxParts; ++p) parts->ptr[p] = parts->ptr[W->n_parts - 1];
  if (n < 1) return fail(AWQ_EINVAL, "group has no rows");
  *d_out = n;
  return AWQ_OK;
}

static size_t wmean_ws(int64_t d_out, int64_t d_in) {
  return align256((size_t)d_out * sizeof(float)) + align256((size_t)wmean_splits(d_out) * d_in * sizeof(double));
}

awq_status awq_weight_channel_mean_workspace(int64_t d_out_total, int64_t d_in, size_t* bytes) {
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (d_out_total < 1 || d_in < 1) return fail(AWQ_EINVAL, "need d_out_total >= 1 and d_in >= 1");
  *bytes = wmean_ws(d_out_total, d_in);
  return ok();
}

awq_status awq_weight_channel_mean(const awq_wgroup* W, int64_t d_in, float* w_mean, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  WParts parts;
  int64_t d_out = 0;
  awq_status st = read_group(W, &parts, &d_out);
  if (st) return st;
  if (d_in < 8 || d_in % 8) return fail(AWQ_ESHAPE, "d_in %lld not a positive multiple of 8", (long long)d_in);
  if (!w_mean) return fail(AWQ_EINVAL, "w_mean is NULL");
  const size_t need = wmean_ws(d_out, d_in);
  if (!ws || ws_bytes < need) return fail(AWQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255u) return fail(AWQ_EALIGN, "ws not 256-byte aligned");
  char* base = (char*)ws;
  return hip_status(launch_weight_channel_mean(parts, d_out, d_in, (float*)base,
                                               (double*)(base + align256((size_t)d_out * sizeof(float))), w_mean,
                                               (hipStream_t)stream),
                    "awq_weight_channel_mean");
}

static size_t duo_cand_ws(int64_t d_in, int n_grid) {
  return align256((size_t)n_grid * d_in * sizeof(double)) +
         align256((size_t)n_grid * duo_cand_blocks(d_in) * 2 * sizeof(double));
}

awq_status awq_candidate_scales_duo_workspace(int64_t d_in, int32_t n_grid, size_t* bytes) {
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (d_in < 1) return fail(AWQ_EINVAL, "d_in must be >= 1");
  if (n_grid < 1 || n_grid > kMaxGrid) return fail(AWQ_EINVAL, "n_grid %d not in [1,%d]", n_grid, kMaxGrid);
  *bytes = duo_cand_ws(d_in, n_grid);
  return ok();
}

awq_status awq_candidate_scales_duo(const float* x_mean, const float* w_mean, int64_t d_in, int32_t n_grid,
                                    double s_min, float* S, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!x_mean || !w_mean || !S) return fail(AWQ_EINVAL, "x_mean / w_mean / S is NULL");
  if (d_in < 1) return fail(AWQ_EINVAL, "d_in must be >= 1");
  if (n_grid < 1 || n_grid > kMaxGrid) return fail(AWQ_EINVAL, "n_grid %d not in [1,%d]", n_grid, kMaxGrid);
  if (!(s_min > 0.0 && isfinite(s_min))) return fail(AWQ_EINVAL, "s_min must be positive and finite");
  const size_t need = duo_cand_ws(d_in, n_grid);
  if (!ws || ws_bytes < need) return fail(AWQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255u) return fail(AWQ_EALIGN, "ws not 256-byte aligned");
  char* base = (char*)ws;
  return hip_status(launch_candidates_duo(x_mean, w_mean, d_in, n_grid, s_min, (double*)base,
                                          (double*)(base + align256((size_t)n_grid * d_in * sizeof(double))), S,
                                          nullptr, (hipStream_t)stream),
                    "awq_candidate_scales_duo");
}

// ---------------------------------------------------------------------------
awq_status awq_search_workspace(const awq_search_cfg* cfg, int64_t d_out_total, int64_t d_in, int64_t T,
                                size_t* bytes) {
  awq_status st = check_cfg(cfg);
  if (st) return st;
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (d_out_total < 1 || d_in < 1) return fail(AWQ_EINVAL, "need d_out_total >= 1 and d_in >= 1");
  if (d_in % cfg->group_size) return fail(AWQ_ESHAPE, "d_in %lld not a multiple of group_size %d", (long long)d_in, cfg->group_size);
  if (cfg->score == AWQ_SCORE_OUTPUT && T < 1) return fail(AWQ_EINVAL, "output score needs T >= 1");
  *bytes = plan_search(*cfg, d_out_total, d_in, T).total;
  return ok();
}

awq_status awq_search_output_form(const awq_search_cfg* cfg, int64_t d_out_total, int64_t d_in, int64_t T,
                                  int32_t* form) {
  awq_status st = check_cfg(cfg);
  if (st) return st;
  if (!form) return fail(AWQ_EINVAL, "form is NULL");
  if (cfg->score != AWQ_SCORE_OUTPUT) return fail(AWQ_EINVAL, "the form applies to the output score only");
  if (d_out_total < 1 || d_in < 1) return fail(AWQ_EINVAL, "need d_out_total >= 1 and d_in >= 1");
  if (d_in % cfg->group_size) return fail(AWQ_ESHAPE, "d_in %lld not a multiple of group_size %d", (long long)d_in, cfg->group_size);
  if (T < 1) return fail(AWQ_EINVAL, "output score needs T >= 1");
  const SearchPlan p = plan_search(*cfg, d_out_total, d_in, T);
  *form = (p.gram ? AWQ_OUT_FORM_GRAM : AWQ_OUT_FORM_DIRECT) | (p.clip_gram ? AWQ_OUT_FORM_CLIP_GRAM : 0);
  return ok();
}

awq_status awq_search_scales(const awq_search_cfg* cfg, const awq_wgroup* W, int64_t d_in,
                             const float* x_mean, const void* X, int32_t x_dtype, int64_t T,
                             int64_t ld_x, float* err, int32_t* best_idx, float* best_s, float* clip,
                             float* clip_err, void* ws, size_t ws_bytes, hipStream_t stream) {
  awq_status st = check_cfg(cfg);
  if (st) return st;
  if (!W || !W->w || !W->rows) return fail(AWQ_EINVAL, "weight group is NULL");
  if (W->n_parts < 1 || W->n_parts > kMaxParts) return fail(AWQ_EINVAL, "n_parts %d not in [1,%d]", W->n_parts, kMaxParts);
  WParts parts{};
  parts.n = W->n_parts;
  int64_t d_out = 0;
  for (int p = 0; p < W->n_parts; ++p) {
    if (W->rows[p] < 0) return fail(AWQ_EINVAL, "rows[%d] < 0", p);
    if (W->rows[p] > 0 && !W->w[p]) return fail(AWQ_EINVAL, "w[%d] is NULL", p);
    if (!aligned16(W->w[p])) return fail(AWQ_EALIGN, "w[%d] not 16-byte aligned", p);
    parts.ptr[p] = (const uint16_t*)W->w[p];
    parts.row_start[p] = d_out;
    d_out += W->rows[p];
  }
  for (int p = W->n_parts; p <= kMaxParts; ++p) parts.row_start[p] = d_out;
  for (int p = W->n_parts; p < kMaxParts; ++p) parts.ptr[p] = parts.ptr[W->n_parts - 1];
  if (d_out < 1) return fail(AWQ_EINVAL, "group has no rows");
  if (d_in < cfg->group_size || d_in % cfg->group_size)
    return fail(AWQ_ESHAPE, "d_in %lld not a positive multiple of group_size %d", (long long)d_in, cfg->group_size);
  if (!x_mean || !err || !best_idx || !best_s) return fail(AWQ_EINVAL, "x_mean / err / best_idx / best_s is NULL");
  if (!aligned16(x_mean) || !aligned16(best_s)) return fail(AWQ_EALIGN, "x_mean / best_s not 16-byte aligned");
  const bool need_x = cfg->score == AWQ_SCORE_OUTPUT || cfg->n_clip >= 2;
  if (need_x) {
    if (!X) return fail(AWQ_EINVAL, "X is NULL (needed by the output score)");
    if (x_dtype != AWQ_F16 && x_dtype != AWQ_BF16) return fail(AWQ_EDTYPE, "x_dtype %d: need AWQ_F16 or AWQ_BF16", x_dtype);
    if (T < 1) return fail(AWQ_EINVAL, "output score needs T >= 1");
    if (ld_x < d_in) return fail(AWQ_ESHAPE, "ld_x %lld < d_in %lld", (long long)ld_x, (long long)d_in);
    if (!aligned16(X) || (ld_x % 8)) return fail(AWQ_EALIGN, "X must be 16-byte aligned with ld_x % 8 == 0");
    // the matrix-core operands are addressed with 32-bit byte offsets
    int64_t tp, dp, kp;
    gemm_sq_pad(T, d_out, d_in, &tp, &dp, &kp);
    if ((double)tp * (double)kp * 2.0 >= 4294967296.0 || (double)dp * (double)kp * 2.0 * 2.0 >= 4294967296.0)
      return fail(AWQ_ESHAPE, "output score needs T*d_in and d_out*d_in below 2^31 elements");
  }
  if (cfg->n_clip >= 2 && !clip) return fail(AWQ_EINVAL, "clip is NULL but n_clip >= 2");
  const SearchPlan plan = plan_search(*cfg, d_out, d_in, T);
  if (plan.output && plan.need_h && !gram_fits(plan))
    return fail(AWQ_ESHAPE, "second-moment output score needs d_in^2 and T*d_in below 2^31 elements");
  if (!ws || ws_bytes < plan.total) return fail(AWQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, plan.total);
  if ((uintptr_t)ws & 255u) return fail(AWQ_EALIGN, "ws not 256-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  float* S = (float*)(base + plan.off_S);
  const bool asym = (cfg->flags & AWQ_FLAG_ASYM) != 0;
  hipError_t e;
  if (!plan.output) {
    float* C2 = (float*)(base + plan.off_C2);
    float* part = (float*)(base + plan.off_part);
    if ((e = launch_cands(*cfg, plan, parts, d_out, d_in, x_mean, base, S, C2, s)) != hipSuccess)
      return hip_status(e, "candidates");
    mark(true, s);
    e = launch_search_weight(cfg->group_size, asym, parts, d_out, d_in, cfg->n_grid, S, C2, part, s);
    mark(false, s);
    if (e != hipSuccess) return hip_status(e, "search_weight");
    if ((e = launch_select(part, plan.n_blocks, cfg->n_grid, 1.0, nullptr, (double*)(base + plan.off_tot), err,
                           best_idx, S, d_in, best_s, s)) != hipSuccess)
      return hip_status(e, "select");
    return ok();
  }

  const bool bf16 = x_dtype == AWQ_BF16;
  uint16_t* x16 = (uint16_t*)(base + plan.off_x16);
  uint16_t* dw = (uint16_t*)(base + plan.off_dw);
  float* colpart = (float*)(base + plan.off_part);
  float* xmax = (float*)(base + plan.off_xmax);
  float* dmax = (float*)(base + plan.off_dmax);
  double* tot = (double*)(base + plan.off_tot);
  OutScales* sc_a = (OutScales*)(base + plan.off_sc);
  OutScales* sc_c = (OutScales*)(base + plan.off_sc + align256(sizeof(OutScales)));
  const int G = cfg->group_size;
  const int64_t dop = plan.d_out_pad, kp = plan.K_pad;
  // second-moment form: H = X^T X once, dW columns scaled by hc = sqrt(diag H)
  const float* hc = plan.need_h ? (const float*)(base + plan.off_hc) : nullptr;
  const uint16_t* h16 = plan.need_h ? (const uint16_t*)(base + plan.off_h16) : nullptr;
  // the alpha search's sums over rows take H'' in fp16; the clip search's
  // per-row forms take it as hi + lo
  auto product = [&](bool gram, bool split, int64_t n_cols, float* part) -> hipError_t {
    return gram ? launch_gemm_gram(h16, plan.g_h_rows, kp, dw, n_cols, part, plan.ldc, split, s)
                : launch_gemm_sq(x16, plan.T_pad, kp, dw, n_cols, part, plan.ldc, s);
  };
  const float* hc_a = plan.gram ? hc : nullptr;
  const float* hc_c = plan.clip_gram ? hc : nullptr;
  if ((e = launch_cands(*cfg, plan, parts, d_out, d_in, x_mean, base, S, nullptr, s)) != hipSuccess)
    return hip_status(e, "candidates");
  if ((e = launch_prepare_x(X, bf16, T, d_in, ld_x, xmax, s)) != hipSuccess) return hip_status(e, "absmax(X)");
  if (plan.need_h) {
    uint16_t* xt = (uint16_t*)(base + plan.off_xt);
    if ((e = launch_out_scales(xmax, plan.n_x, nullptr, 0, 1, sc_a, s)) != hipSuccess)
      return hip_status(e, "out_scales(X)");
    if ((e = launch_transpose_x(X, bf16, T, d_in, ld_x, plan.g_T_pad, plan.g_xt_rows, sc_a, xt, s)) != hipSuccess)
      return hip_status(e, "transpose_x");
    float* h32 = (float*)(base + plan.off_h32);
    if ((e = launch_gemm_gram_h(xt, plan.g_T_pad, kp, h32, s)) != hipSuccess) return hip_status(e, "gemm(H)");
    if ((e = launch_gram_scale(h32, plan.g_T_pad, kp, plan.g_h_rows, (float*)(base + plan.off_hc),
                               (float*)(base + plan.off_hr), (uint16_t*)h16, s)) != hipSuccess)
      return hip_status(e, "gram_scale");
  }
  float* cmax = (float*)(base + plan.off_cmax);
  if ((e = launch_colmax(parts, d_out, d_in, (float*)(base + plan.off_cpart), cmax, s)) != hipSuccess)
    return hip_status(e, "colmax");
  if ((e = launch_dw_bound(asym, cmax, d_in, cfg->n_grid, 0, S, nullptr, 0, 1.0f, hc_a, dmax, s)) != hipSuccess)
    return hip_status(e, "dw_bound");
  if ((e = launch_out_scales(xmax, plan.n_x, dmax, plan.n_db, cfg->n_grid, sc_a, s)) != hipSuccess)
    return hip_status(e, "out_scales");
  if (plan.need_x16 && (e = launch_convert_x(X, bf16, T, d_in, ld_x, plan.T_pad, kp, sc_a, x16, s)) != hipSuccess)
    return hip_status(e, "convert_x");
  const bool one_chunk = plan.cand_chunk >= cfg->n_grid;
  if (!one_chunk) mark(true, s);
  for (int c0 = 0; c0 < cfg->n_grid; c0 += plan.cand_chunk) {
    const int nc = (cfg->n_grid - c0) < plan.cand_chunk ? (cfg->n_grid - c0) : plan.cand_chunk;
    if ((e = launch_build_dw(G, asym, parts, d_out, d_in, dop, kp, nc, 0, S, nullptr, 0, 1.0f, c0, sc_a, hc_a, dw, s)) !=
        hipSuccess)
      return hip_status(e, "build_dw");
    if (one_chunk) mark(true, s);
    e = product(plan.gram, false, (int64_t)nc * dop, colpart + (int64_t)c0 * dop);
    if (one_chunk) mark(false, s);
    if (e != hipSuccess) return hip_status(e, "gemm_sq");
  }
  if (!one_chunk) mark(false, s);
  double* chunk_sum = (double*)(base + plan.off_chunk);
  const int64_t nch = reduce_cols_chunks(d_out);
  if ((e = launch_reduce_cols(colpart, plan.n_mt_a, plan.ldc, d_out, dop, cfg->n_grid, chunk_sum, s)) != hipSuccess)
    return hip_status(e, "reduce_cols");
  if ((e = launch_select(chunk_sum, nch, cfg->n_grid, 1.0 / ((double)T * (double)d_out), sc_a->inv, tot, err,
                         best_idx, S, d_in, best_s, s)) != hipSuccess)
    return hip_status(e, "select");
  if (cfg->n_clip >= 2) {
    const int nclip = cfg->n_clip;
    if ((e = launch_dw_bound(asym, cmax, d_in, nclip, 1, nullptr, best_s, nclip, cfg->clip_lo, hc_c, dmax, s)) !=
        hipSuccess)
      return hip_status(e, "dw_bound(clip)");
    if ((e = launch_out_scales(xmax, plan.n_x, dmax, plan.n_db, nclip, sc_c, s)) != hipSuccess)
      return hip_status(e, "out_scales(clip)");
    for (int c0 = 0; c0 < nclip; c0 += plan.cand_chunk) {
      const int nc = (nclip - c0) < plan.cand_chunk ? (nclip - c0) : plan.cand_chunk;
      if ((e = launch_build_dw(G, asym, parts, d_out, d_in, dop, kp, nc, 1, nullptr, best_s, nclip, cfg->clip_lo, c0,
                               sc_c, hc_c, dw, s)) != hipSuccess)
        return hip_status(e, "build_dw(clip)");
      if ((e = product(plan.clip_gram, true, (int64_t)nc * dop, colpart + (int64_t)c0 * dop)) != hipSuccess)
        return hip_status(e, "gemm_sq(clip)");
    }
    if ((e = launch_clip_select(colpart, plan.n_mt_c, plan.ldc, d_out, dop, nclip, cfg->clip_lo, sc_c, clip, clip_err,
                                s)) != hipSuccess)
      return hip_status(e, "clip_select");
  }
  return ok();
}

// ---------------------------------------------------------------------------
// Weight-score search without a caller workspace: the scratch lives in a
// file-scope device array (one copy per GPU, kept until the process ends).
// Host code never uses the array's name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch (set up on first use)
awq_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(AWQ_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(AWQ_EINVAL, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(AWQ_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}
}  // namespace

extern "C" awq_status awq_search_scales_noalloc(const awq_search_cfg* cfg, const awq_wgroup* W, int64_t d_in,
                                                const float* x_mean, float* err, int32_t* best_idx, float* best_s,
                                                hipStream_t stream) {
  awq_status st = check_cfg(cfg);
  if (st) return st;
  if (cfg->score != AWQ_SCORE_WEIGHT || cfg->n_clip != 0)
    return fail(AWQ_EINVAL, "awq_search_scales_noalloc: weight score only (no output score, no clip search)");
  WParts parts;
  int64_t d_out = 0;
  if ((st = read_group(W, &parts, &d_out))) return st;
  if (d_in < cfg->group_size || d_in % cfg->group_size)
    return fail(AWQ_ESHAPE, "d_in %lld not a positive multiple of group_size %d", (long long)d_in, cfg->group_size);
  const size_t need = plan_search(*cfg, d_out, d_in, 0).total;
  if (need > kNoAllocScratchBytes)
    return fail(AWQ_EWORKSPACE, "awq_search_scales_noalloc: this search needs %zu bytes of scratch, more than the "
                "library's %zu", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((st = device_scratch(&ws))) return st;
  return awq_search_scales(cfg, W, d_in, x_mean, nullptr, AWQ_BF16, 0, 0, err, best_idx, best_s, nullptr, nullptr,
                           ws, kNoAllocScratchBytes, stream);
}

// ---------------------------------------------------------------------------
static awq_status quantize_pack_impl(const void* W, int64_t d_out, int64_t d_in, int32_t group_size, bool asym,
                                     const float* s, const float* clip, int32_t* qweight, uint16_t* scales,
                                     int32_t* qzeros, hipStream_t stream, const char* name) {
  if (!valid_group(group_size)) return fail(AWQ_EINVAL, "group_size %d not in {32,64,128}", group_size);
  if (d_out < 0 || d_in < 0) return fail(AWQ_EINVAL, "negative size");
  if (d_out % 8) return fail(AWQ_ESHAPE, "d_out %lld not a multiple of 8", (long long)d_out);
  if (d_in % group_size) return fail(AWQ_ESHAPE, "d_in %lld not a multiple of group_size %d", (long long)d_in, group_size);
  if (d_out == 0 || d_in == 0) return ok();
  if (!W || !qweight || !scales) return fail(AWQ_EINVAL, "W / qweight / scales is NULL");
  if (asym && !qzeros) return fail(AWQ_EINVAL, "qzeros is NULL (asymmetric zero points are data)");
  if (!aligned16(W) || !aligned16(scales)) return fail(AWQ_EALIGN, "W / scales not 16-byte aligned");
  if (s && !aligned16(s)) return fail(AWQ_EALIGN, "s not 16-byte aligned");
  if (((uintptr_t)qweight & 3u) || (qzeros && ((uintptr_t)qzeros & 3u)) || (clip && ((uintptr_t)clip & 3u)))
    return fail(AWQ_EALIGN, "qweight / qzeros / clip not 4-byte aligned");
  mark(true, (hipStream_t)stream);
  hipError_t e = launch_quantize_pack((const uint16_t*)W, d_out, d_in, group_size, asym, s, clip, qweight, scales,
                                      qzeros, (hipStream_t)stream);
  mark(false, (hipStream_t)stream);
  return hip_status(e, name);
}

awq_status awq_quantize_pack(const void* W, int64_t d_out, int64_t d_in, int32_t group_size, const float* s,
                             const float* clip, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                             hipStream_t stream) {
  return quantize_pack_impl(W, d_out, d_in, group_size, false, s, clip, qweight, scales, qzeros, stream,
                            "awq_quantize_pack");
}

awq_status awq_quantize_pack_asym(const void* W, int64_t d_out, int64_t d_in, int32_t group_size, const float* s,
                                  const float* clip, int32_t* qweight, uint16_t* scales, int32_t* qzeros,
                                  hipStream_t stream) {
  return quantize_pack_impl(W, d_out, d_in, group_size, true, s, clip, qweight, scales, qzeros, stream,
                            "awq_quantize_pack_asym");
}

// ---------------------------------------------------------------------------
static int w4a16_mt(int64_t M) { return M >= 3 ? 4 : (int)M; }

awq_status awq_w4a16_workspace(int64_t M, int64_t d_out, int64_t d_in, size_t* bytes) {
  if (!bytes) return fail(AWQ_EINVAL, "bytes is NULL");
  if (M < 0 || d_out < 0 || d_in < 0) return fail(AWQ_EINVAL, "negative size");
  const size_t gemv = (size_t)w4a16_slices(d_in) * (size_t)w4a16_mt(M) * (size_t)d_out;
  const size_t gemm = (size_t)w4a16_gemm_part_floats(M, d_out, d_in);
  const size_t skinny =   // the few-token path's input ranges
      (d_out > 0 && d_in > 0) ? (size_t)w4a16_skinny_part_floats(M, d_out, d_in) : 0;
  size_t need = gemv > gemm ? gemv : gemm;
  need = need > skinny ? need : skinny;
  *bytes = align256(need * sizeof(float));
  return ok();
}

awq_status awq_w4a16_matmul(const void* X, int64_t M, int64_t ld_x, const int32_t* qweight, const uint16_t* scales,
                            const int32_t* qzeros, int64_t d_out, int64_t d_in, int32_t group_size, void* Y,
                            int64_t ld_y, int32_t y_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_group(group_size)) return fail(AWQ_EINVAL, "group_size %d not in {32,64,128}", group_size);
  if (M < 0 || d_out < 0 || d_in < 0) return fail(AWQ_EINVAL, "negative size");
  if (d_out % 8) return fail(AWQ_ESHAPE, "d_out %lld not a multiple of 8", (long long)d_out);
  if (d_in % group_size) return fail(AWQ_ESHAPE, "d_in %lld not a multiple of group_size %d", (long long)d_in, group_size);
  if (y_dtype != AWQ_F16 && y_dtype != AWQ_F32) return fail(AWQ_EDTYPE, "y_dtype %d: need AWQ_F16 or AWQ_F32", y_dtype);
  if (M == 0 || d_out == 0) return ok();
  if (d_in == 0) return fail(AWQ_ESHAPE, "d_in is 0 with M, d_out > 0");
  if (ld_x < d_in) return fail(AWQ_ESHAPE, "ld_x %lld < d_in %lld", (long long)ld_x, (long long)d_in);
  if (ld_y < d_out || ld_y % 4) return fail(AWQ_ESHAPE, "ld_y %lld: need >= d_out and a multiple of 4", (long long)ld_y);
  if (!X || !qweight || !scales || !Y) return fail(AWQ_EINVAL, "X / qweight / scales / Y is NULL");
  if (((uintptr_t)X & 1u) || ((uintptr_t)qweight & 3u) || (qzeros && ((uintptr_t)qzeros & 3u)))
    return fail(AWQ_EALIGN, "X / qweight / qzeros misaligned");
  if (!aligned16(scales)) return fail(AWQ_EALIGN, "scales not 16-byte aligned");
  if ((uintptr_t)Y & (y_dtype == AWQ_F16 ? 7u : 15u)) return fail(AWQ_EALIGN, "Y misaligned for vector stores");
  size_t need = 0;
  awq_w4a16_workspace(M, d_out, d_in, &need);
  if (!ws || ws_bytes < need) return fail(AWQ_EWORKSPACE, "workspace %zu bytes < %zu", ws_bytes, need);
  if ((uintptr_t)ws & 255u) return fail(AWQ_EALIGN, "ws not 256-byte aligned");
  mark(true, (hipStream_t)stream);
  hipError_t e = launch_w4a16((const uint16_t*)X, M, ld_x, (const uint32_t*)qweight, scales, (const uint32_t*)qzeros,
                              d_out, d_in, group_size, Y, ld_y, y_dtype == AWQ_F16, (float*)ws, (hipStream_t)stream);
  mark(false, (hipStream_t)stream);
  return hip_status(e, "awq_w4a16_matmul");
}

awq_status awq_norm_group_fold(const float* const* s, int32_t n_members, int64_t d_in, const void* norm,
                               int32_t norm_dtype, void* norm_out, float* s_shared, hipStream_t stream) {
  if (!s) return fail(AWQ_EINVAL, "s is NULL");
  if (n_members < 1 || n_members > kMaxParts)
    return fail(AWQ_EINVAL, "n_members %d not in [1,%d]", n_members, kMaxParts);
  if (d_in < 0) return fail(AWQ_EINVAL, "negative size");
  if (norm && norm_dtype != AWQ_F16 && norm_dtype != AWQ_BF16 && norm_dtype != AWQ_F32)
    return fail(AWQ_EDTYPE, "norm_dtype %d: need AWQ_F16, AWQ_BF16 or AWQ_F32", norm_dtype);
  if (norm && !norm_out) return fail(AWQ_EINVAL, "norm given but norm_out is NULL");
  if (!norm && norm_out) return fail(AWQ_EINVAL, "norm_out given but norm is NULL");
  if (d_in == 0) return ok();
  if (!s_shared) return fail(AWQ_EINVAL, "s_shared is NULL");
  ScaleSet S{};
  S.n = n_members;
  for (int m = 0; m < n_members; ++m) {
    if (!s[m]) return fail(AWQ_EINVAL, "s[%d] is NULL", m);
    S.p[m] = s[m];
  }
  for (int m = n_members; m < kMaxParts; ++m) S.p[m] = s[0];
  const size_t esz = norm_dtype == AWQ_F32 ? 4 : 2;
  if (norm && ((uintptr_t)norm % esz || (uintptr_t)norm_out % esz))
    return fail(AWQ_EALIGN, "norm / norm_out not aligned to their element size");
  if ((uintptr_t)s_shared & 3u) return fail(AWQ_EALIGN, "s_shared not 4-byte aligned");
  mark(true, (hipStream_t)stream);
  hipError_t e = launch_norm_group_fold(S, d_in, norm, norm_dtype, norm_out, s_shared, (hipStream_t)stream);
  mark(false, (hipStream_t)stream);
  return hip_status(e, "awq_norm_group_fold");
}

awq_status awq_unpack_dequant(const int32_t* qweight, const uint16_t* scales, const int32_t* qzeros, int64_t d_out,
                              int64_t d_in, int32_t group_size, const float* s, void* out, int32_t out_dtype,
                              hipStream_t stream) {
  if (!valid_group(group_size)) return fail(AWQ_EINVAL, "group_size %d not in {32,64,128}", group_size);
  if (out_dtype != AWQ_F32 && out_dtype != AWQ_F16) return fail(AWQ_EDTYPE, "out_dtype %d: need AWQ_F32 or AWQ_F16", out_dtype);
  if (d_out < 0 || d_in < 0) return fail(AWQ_EINVAL, "negative size");
  if (d_out % 8) return fail(AWQ_ESHAPE, "d_out %lld not a multiple of 8", (long long)d_out);
  if (d_in % group_size) return fail(AWQ_ESHAPE, "d_in %lld not a multiple of group_size %d", (long long)d_in, group_size);
  if (d_out == 0 || d_in == 0) return ok();
  if (!qweight || !scales || !out) return fail(AWQ_EINVAL, "qweight / scales / out is NULL");
  return hip_status(launch_unpack_dequant(qweight, scales, qzeros, d_out, d_in, group_size, s, out,
                                          out_dtype == AWQ_F16, (hipStream_t)stream),
                    "awq_unpack_dequant");
}

}  // extern "C"
