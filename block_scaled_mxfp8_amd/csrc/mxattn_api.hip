// C ABI of libmxattn (declared in include/mxattn.h): host-side validation, sizing and
// kernel launches. Nothing here reads device memory or synchronises, except mx_read_flags.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mxattn.h"
#include "mx_worklist.h"
#include "mx_internal.h"
#include "mx_gemm.h"
#include "mx_norm.h"
#include "mx_layout.h"
#include "mx_profile.h"

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool make_geom(const mx_seq* s, mx::Geom* g) {
  if (!s) return false;
  if (s->cu_seqlens) {
    if (s->n_docs < 1 || s->total_tokens < 0 || s->max_seqlen < 1) return false;
    if (s->total_tokens > (1LL << 31) - 64) return false;
    g->cu = s->cu_seqlens;
    g->batch = 1;
    g->seqlen = 0;
    g->n_docs = s->n_docs;
    g->max_seqlen = s->max_seqlen;
    g->total = s->total_tokens;
    g->gseq = (int)(s->total_tokens / 32 + s->n_docs);
  } else {
    if (s->batch < 1 || s->seqlen < 1 || s->seqlen > (1LL << 30) || s->batch > (1LL << 20)) return false;
    g->cu = nullptr;
    g->batch = (int)s->batch;
    g->seqlen = (int)s->seqlen;
    g->n_docs = (int)s->batch;
    g->max_seqlen = (int)s->seqlen;
    g->total = s->batch * s->seqlen;
    g->gseq = (int)((s->seqlen + 31) / 32);
  }
  return true;
}

size_t row_codes_bytes(const mx::Geom& g, int heads, int d) { return (size_t)g.total * heads * d; }
size_t seq_codes_bytes(const mx::Geom& g, int heads, int d) {
  const size_t rows = mx::packed(g) ? (size_t)g.gseq * heads : (size_t)g.gseq * heads * g.batch;
  return rows * d * 32;
}

bool valid_dim(int d) { return d == 64 || d == 128; }

bool score_fp4(const mx_attn_desc* d) { return d->score_format == MX_SCORE_MXFP4; }

mx_status check_view(const mx_qview& v) {
  if (!v.codes || !v.scales) return MX_E_ARG;
  if (!aligned(v.codes, 16) || !aligned(v.scales, 4)) return MX_E_ARG;
  return MX_OK;
}

mx_status check_desc(const mx_attn_desc* d, mx::Geom* g) {
  if (!d) return MX_E_ARG;
  if (!make_geom(&d->seq, g)) return MX_E_ARG;
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q % d->heads_kv != 0) return MX_E_ARG;
  if (d->out_dtype != MX_F32 && d->out_dtype != MX_BF16) return MX_E_ARG;
  if (!(d->softmax_scale >= 0.f) || !isfinite(d->softmax_scale)) return MX_E_ARG;
  if (d->dq_mode != MX_DQ_F32 && d->dq_mode != MX_DQ_F16_BOOST && d->dq_mode != MX_DQ_F16_PREFIX) return MX_E_ARG;
  if (!valid_dim(d->head_dim)) return MX_E_UNSUPPORTED;
  if (d->deterministic != 0 && d->deterministic != 1) return MX_E_ARG;
  if (d->score_format != MX_SCORE_MXFP8 && d->score_format != MX_SCORE_MXFP4) return MX_E_ARG;
  return MX_OK;
}

// Backward workspace: the status word, G's views, -D and LSE * log2 e (always), then the optional dS code
// store (total_store - total bytes; with it the dQ pass reads dS instead of rebuilding it).
// The kernels index the store's blocks and exponents with 32-bit integers; a geometry whose
// store would need more has no store (store_ok false, total_store = total).
struct BwdWorkspace {
  size_t gr_codes, gr_scales, gs_codes, gs_scales, ndelta, lse2, flags, total;
  size_t gnorm, vpre, kpre;   // prefix dQ boost only (0 otherwise)
  size_t ds_codes, ds_exps, total_store;
  bool store_ok;
  mx::DsStore ds;
};

BwdWorkspace bwd_layout(const mx::Geom& g, const mx::Geom& gk, const mx_attn_desc* d) {
  BwdWorkspace w;
  const int hq = d->heads_q, dim = d->head_dim;
  size_t off = 0;
  w.flags = off; off += align_up(sizeof(uint32_t));   // status word first: mx_read_flags finds it
  w.gr_codes = off; off += align_up(row_codes_bytes(g, hq, dim));
  w.gr_scales = off; off += align_up(row_codes_bytes(g, hq, dim) / 32);
  w.gs_codes = off; off += align_up(seq_codes_bytes(g, hq, dim));
  w.gs_scales = off; off += align_up(seq_codes_bytes(g, hq, dim) / 32);
  w.ndelta = off; off += align_up((size_t)g.total * hq * sizeof(float));
  w.lse2 = off; off += align_up((size_t)g.total * hq * sizeof(float));
  w.gnorm = w.vpre = w.kpre = 0;
  if (d->dq_mode == MX_DQ_F16_PREFIX) {   // |G~| per (row, head), prefix maxima per (key, KV head)
    w.gnorm = off; off += align_up((size_t)g.total * hq * sizeof(float));
    w.vpre = off; off += align_up((size_t)gk.total * d->heads_kv * sizeof(float));
    w.kpre = off; off += align_up((size_t)gk.total * d->heads_kv * sizeof(float));
  }
  w.total = off;
  w.ds = mx::ds_store_geom(g, gk, d->causal != 0);
  const size_t rows = (size_t)g.gseq * hq * (mx::packed(g) ? 1 : (size_t)g.batch);   // query groups
  const size_t blocks = w.ds.tri ? (size_t)g.batch * hq * (size_t)w.ds.head_blocks : rows * (size_t)w.ds.cols;
  w.store_ok = blocks <= UINT32_MAX && rows * (size_t)w.ds.ecols <= UINT32_MAX;
  w.ds_codes = off; off += align_up(blocks * 1024);
  w.ds_exps = off; off += align_up(rows * (size_t)w.ds.ecols);
  w.total_store = w.store_ok ? off : w.total;
  return w;
}

// Key geometry of a call: the queries' own for self-attention (seq_k == nullptr); for
// cross-attention *seq_k, which must use the same layout (batched with the same batch, or
// packed with the same number of documents: document j's queries attend to document j's
// keys). Cross-attention is non-causal.
mx_status key_geom(const mx_attn_desc* d, const mx::Geom& g, const mx_seq* seq_k, mx::Geom* gk) {
  if (!seq_k) {
    *gk = g;
    return MX_OK;
  }
  if (!make_geom(seq_k, gk)) return MX_E_ARG;
  if (mx::packed(g) != mx::packed(*gk)) return MX_E_ARG;
  if (mx::packed(g) ? gk->n_docs != g.n_docs : gk->batch != g.batch) return MX_E_ARG;
  if (d->causal) return MX_E_UNSUPPORTED;
  return MX_OK;
}

mx_status fwd_impl(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview k_row, mx_qview v_seq,
                   void* o, float* lse, void* stream, bool need_packed, const mx_qview* v_tok = nullptr) {
  mx::Geom g, gk;
  mx_status st = check_desc(desc, &g);
  if (st != MX_OK) return st;
  if (need_packed && !desc->seq.cu_seqlens) return MX_E_ARG;
  if ((st = key_geom(desc, g, seq_k, &gk)) != MX_OK) return st;
  if ((st = check_view(q_row)) != MX_OK || (st = check_view(k_row)) != MX_OK || (st = check_view(v_seq)) != MX_OK)
    return st;
  if (!o || !lse || !aligned(o, 16) || !aligned(lse, 4)) return MX_E_ARG;
  if (v_tok) {   // the strict per-key V fold: causal self-attention with E4M3 scores
    if ((st = check_view(*v_tok)) != MX_OK) return st;
    if (!desc->causal || seq_k) return MX_E_ARG;
    if (score_fp4(desc)) return MX_E_UNSUPPORTED;
  }
  mx::AttnParams p = {};
  p.geom = g;
  p.geom_k = gk;
  p.heads_q = desc->heads_q;
  p.heads_kv = desc->heads_kv;
  p.head_dim = desc->head_dim;
  p.causal = desc->causal ? 1 : 0;
  p.scale = desc->softmax_scale > 0.f ? desc->softmax_scale : 1.0f / sqrtf((float)desc->head_dim);
  p.out_f32 = desc->out_dtype == MX_F32;
  p.plan = mx::plan_eligible(g, gk) ? 1 : 0;
  p.score_fp4 = score_fp4(desc);
  p.q_codes = q_row.codes; p.q_scales = q_row.scales;
  p.k_codes = k_row.codes; p.k_scales = k_row.scales;
  p.v_codes = v_seq.codes; p.v_scales = v_seq.scales;
  if (v_tok) {
    p.vt_codes = v_tok->codes;
    p.vt_scales = v_tok->scales;
  }
  p.o = o;
  p.lse = lse;
  if (g.total == 0) return MX_OK;
  return mx::launch_attn_fwd(p, (hipStream_t)stream) == hipSuccess ? MX_OK : MX_E_DEVICE;
}

mx_status bwd_impl(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                   mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* gptr, mx_dtype g_dtype,
                   void* dq, void* dk, void* dv, void* stream, bool need_packed, const mx_qview* mx_out = nullptr,
                   const mx_qview* k_tok = nullptr) {
  mx::Geom g, gk;
  mx_status st = check_desc(desc, &g);
  if (st != MX_OK) return st;
  if (need_packed && !desc->seq.cu_seqlens) return MX_E_ARG;
  if ((st = key_geom(desc, g, seq_k, &gk)) != MX_OK) return st;
  const mx_qview views[5] = {q_row, q_seq, k_row, k_seq, v_row};
  for (const auto& v : views)
    if ((st = check_view(v)) != MX_OK) return st;
  if (!o || !lse || !gptr || !dq || !dk || !dv) return MX_E_ARG;
  if (!aligned(o, 16) || !aligned(gptr, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16)) return MX_E_ARG;
  if (g_dtype != MX_F32 && g_dtype != MX_BF16) return MX_E_ARG;
  if (k_tok) {   // the strict dQ: causal self-attention, FP32 dQ, E4M3 scores
    if ((st = check_view(*k_tok)) != MX_OK) return st;
    if (!desc->causal || seq_k) return MX_E_ARG;
    if (desc->dq_mode != MX_DQ_F32 || score_fp4(desc)) return MX_E_UNSUPPORTED;
  }
  const BwdWorkspace w = bwd_layout(g, gk, desc);
  if (!desc->workspace || desc->workspace_bytes < w.total || !aligned(desc->workspace, kAlign)) return MX_E_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(desc->workspace);
  mx::BwdParams p = {};
  p.geom = g;
  p.geom_k = gk;
  p.heads_q = desc->heads_q;
  p.heads_kv = desc->heads_kv;
  p.head_dim = desc->head_dim;
  p.causal = desc->causal ? 1 : 0;
  p.scale = desc->softmax_scale > 0.f ? desc->softmax_scale : 1.0f / sqrtf((float)desc->head_dim);
  p.out_f32 = desc->out_dtype == MX_F32;
  p.plan = mx::plan_eligible(g, gk) ? 1 : 0;
  p.score_fp4 = score_fp4(desc);
  p.dq_mode = desc->dq_mode;
  p.q_codes = q_row.codes; p.q_scales = q_row.scales;
  p.qs_codes = q_seq.codes; p.qs_scales = q_seq.scales;
  p.k_codes = k_row.codes; p.k_scales = k_row.scales;
  p.ks_codes = k_seq.codes; p.ks_scales = k_seq.scales;
  p.vr_codes = v_row.codes; p.vr_scales = v_row.scales;
  p.o = o;
  p.lse = lse;
  p.g = gptr;
  p.g_f32 = g_dtype == MX_F32;
  p.dq = dq; p.dk = dk; p.dv = dv;
  p.gr_codes = ws + w.gr_codes; p.gr_scales = ws + w.gr_scales;
  p.gs_codes = ws + w.gs_codes; p.gs_scales = ws + w.gs_scales;
  p.ndelta = reinterpret_cast<float*>(ws + w.ndelta);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.flags = reinterpret_cast<uint32_t*>(ws + w.flags);
  if (desc->dq_mode == MX_DQ_F16_PREFIX) {
    p.gnorm = reinterpret_cast<float*>(ws + w.gnorm);
    p.vpre = reinterpret_cast<float*>(ws + w.vpre);
    p.kpre = reinterpret_cast<float*>(ws + w.kpre);
  }
  if (k_tok) {   // (dQ rebuilds its own per-query dS, so the code store is not used)
    p.kt_codes = k_tok->codes;
    p.kt_scales = k_tok->scales;
  } else if (w.store_ok && desc->workspace_bytes >= w.total_store) {
    p.ds_codes = ws + w.ds_codes;
    p.ds_exps = ws + w.ds_exps;
    p.ds = w.ds;
  } else if (p.score_fp4) {
    // the 4-bit score path has only the dK/dV kernel rebuild S: dQ reads the stored dS codes
    return w.store_ok ? MX_E_WORKSPACE : MX_E_UNSUPPORTED;
  }
  if (mx_out) {   // dK ROW, dK SEQ, dV ROW, dV SEQ; a view with null codes is not wanted
    const mx_qview& a = mx_out[0];
    const mx_qview& b = mx_out[1];
    const mx_qview& c = mx_out[2];
    const mx_qview& d = mx_out[3];
    for (int i = 0; i < 4; i++)
      if (mx_out[i].codes && check_view(mx_out[i]) != MX_OK) return MX_E_ARG;
    p.dkr_codes = a.codes; p.dkr_scales = a.codes ? a.scales : nullptr;
    p.dks_codes = b.codes; p.dks_scales = b.codes ? b.scales : nullptr;
    p.dvr_codes = c.codes; p.dvr_scales = c.codes ? c.scales : nullptr;
    p.dvs_codes = d.codes; p.dvs_scales = d.codes ? d.scales : nullptr;
  }
  if (g.total == 0) return MX_OK;
  return mx::launch_attn_bwd(p, (hipStream_t)stream) == hipSuccess ? MX_OK : MX_E_DEVICE;
}

// Library-owned scratch of mx_attn_bwd_noalloc: the minimal backward workspace (G views, -D,
// LSE log2 e, the status word) for callers that cannot allocate. One copy per device, alive
// until the process ends. Host code never uses the array's name as an address: it is a
// host-side stand-in; the device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (null: not yet looked up)

// Device address of the current device's scratch (looked up on the first call on a device,
// with that device current).
mx_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MX_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MX_E_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MX_OK;
}

}  // namespace

namespace mx {
ProfileHook& profile_hook() {
  static ProfileHook hook;
  return hook;
}
}  // namespace mx

extern "C" {

static mx_status quantize_impl(const mx_seq* seq, int32_t heads, int32_t head_dim, const void* x, mx_dtype dtype,
                               int32_t views, mx_qview* row_out, mx_qview* seq_out, void* stream, bool token_block) {
  mx::Geom g;
  if (!make_geom(seq, &g) || heads < 1 || !x) return MX_E_ARG;
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_E_ARG;
  if (views < 1 || views > (MX_VIEW_SEQ | MX_VIEW_ROW_FP4 | MX_VIEW_SEQ_TOKEN)) return MX_E_ARG;
  if ((views & MX_VIEW_ROW) && (views & MX_VIEW_ROW_FP4)) return MX_E_ARG;        // one row_out
  if ((views & MX_VIEW_SEQ) && (views & MX_VIEW_SEQ_TOKEN)) return MX_E_ARG;      // one seq_out
  if (!valid_dim(head_dim)) return MX_E_UNSUPPORTED;
  if (token_block && (views & (MX_VIEW_ROW_FP4 | MX_VIEW_SEQ_TOKEN))) return MX_E_UNSUPPORTED;
  if (!aligned(x, 16)) return MX_E_ARG;
  mx::QuantizeParams p = {};
  p.geom = g;
  p.heads = heads;
  p.head_dim = head_dim;
  p.f32 = dtype == MX_F32;
  p.token_block = token_block;
  p.x = x;
  if (views & (MX_VIEW_ROW | MX_VIEW_ROW_FP4)) {
    if (!row_out || check_view(*row_out) != MX_OK) return MX_E_ARG;
    p.row_codes = row_out->codes;
    p.row_scales = row_out->scales;
    p.row_fp4 = (views & MX_VIEW_ROW_FP4) != 0;
  }
  if (views & (MX_VIEW_SEQ | MX_VIEW_SEQ_TOKEN)) {
    if (!seq_out || check_view(*seq_out) != MX_OK) return MX_E_ARG;
    p.seq_codes = seq_out->codes;
    p.seq_scales = seq_out->scales;
    p.seq_token = (views & MX_VIEW_SEQ_TOKEN) != 0;
  }
  if (g.total == 0) return MX_OK;
  const int slot = mx::profile_begin(mx::kProfQuantize, (hipStream_t)stream);
  const hipError_t err = mx::launch_quantize(p, (hipStream_t)stream);
  mx::profile_end(slot, (hipStream_t)stream);
  return err == hipSuccess ? MX_OK : MX_E_DEVICE;
}

mx_status mx_quantize(const mx_seq* seq, int32_t heads, int32_t head_dim, const void* x, mx_dtype dtype, int32_t views,
                      mx_qview* row_out, mx_qview* seq_out, void* stream) {
  return quantize_impl(seq, heads, head_dim, x, dtype, views, row_out, seq_out, stream, false);
}

mx_status mx_quantize_token_block(const mx_seq* seq, int32_t heads, int32_t head_dim, const void* x, mx_dtype dtype,
                                  int32_t views, mx_qview* row_out, mx_qview* seq_out, void* stream) {
  return quantize_impl(seq, heads, head_dim, x, dtype, views, row_out, seq_out, stream, true);
}

mx_status mx_rmsnorm_quantize(const void* x, const void* gamma, mx_dtype dtype, int64_t rows, int32_t n, float eps,
                              int32_t views, mx_qview* row_out, mx_qview* seq_out, void* stream) {
  if (rows < 0 || n < 32 || n % 32 != 0) return MX_E_ARG;
  if (dtype != MX_F32 && dtype != MX_BF16) return MX_E_ARG;
  if (views < 1 || views > 3) return MX_E_ARG;
  if (!(eps >= 0.f) || !(eps <= 3.4e38f)) return MX_E_ARG;   // NaN fails both
  if (n > 65536 || rows > (int64_t)0x7FFFFFFF * 32) return MX_E_UNSUPPORTED;
  if (rows == 0) return MX_OK;          // nothing is read or written: every pointer may be NULL
  if (!x || !gamma || !aligned(x, 16) || !aligned(gamma, 16)) return MX_E_ARG;
  mx::RmsNormParams p = {};
  p.x = x;
  p.gamma = gamma;
  p.f32 = dtype == MX_F32;
  p.rows = rows;
  p.n = n;
  p.eps = eps;
  if (views & MX_VIEW_ROW) {
    if (!row_out || check_view(*row_out) != MX_OK) return MX_E_ARG;
    p.row_codes = row_out->codes;
    p.row_scales = row_out->scales;
  }
  if (views & MX_VIEW_SEQ) {
    if (!seq_out || check_view(*seq_out) != MX_OK) return MX_E_ARG;
    p.seq_codes = seq_out->codes;
    p.seq_scales = seq_out->scales;
  }
  const int slot = mx::profile_begin(mx::kProfRmsNorm, (hipStream_t)stream);
  const hipError_t err = mx::launch_rmsnorm_quantize(p, (hipStream_t)stream);
  mx::profile_end(slot, (hipStream_t)stream);
  return err == hipSuccess ? MX_OK : MX_E_DEVICE;
}

mx_status mx_gemm_quantize(mx_qview a_row, mx_qview b_row, int64_t m, int32_t n, int32_t k, int32_t views,
                           mx_qview* row_out, mx_qview* seq_out, void* stream) {
  if (m < 0 || n < 32 || n % 32 != 0 || k < 64 || k % 64 != 0) return MX_E_ARG;
  if (views < 1 || views > 3) return MX_E_ARG;
  if (m > 0x7FFFFFFF || n > (1 << 24) || k > (1 << 23)) return MX_E_UNSUPPORTED;
  // one 512-thread workgroup per 256 x 256 tile: the grid's work-items must stay below 2^32
  // (this also keeps m + 255 and the tile count inside 32-bit arithmetic in the kernel)
  if (((m + 255) / 256) * (int64_t)((n + 255) / 256) * 512 >= ((int64_t)1 << 32)) return MX_E_UNSUPPORTED;
  if (m == 0) return MX_OK;             // nothing is read or written: every pointer may be NULL
  if (check_view(a_row) != MX_OK || check_view(b_row) != MX_OK) return MX_E_ARG;
  mx::GemmQuantParams p = {};
  p.a_codes = a_row.codes;
  p.a_scales = a_row.scales;
  p.b_codes = b_row.codes;
  p.b_scales = b_row.scales;
  p.m = (int)m;
  p.n = n;
  p.k = k;
  if (views & MX_VIEW_ROW) {
    if (!row_out || check_view(*row_out) != MX_OK) return MX_E_ARG;
    p.row_codes = row_out->codes;
    p.row_scales = row_out->scales;
  }
  if (views & MX_VIEW_SEQ) {
    if (!seq_out || check_view(*seq_out) != MX_OK) return MX_E_ARG;
    p.seq_codes = seq_out->codes;
    p.seq_scales = seq_out->scales;
  }
  const int slot = mx::profile_begin(mx::kProfGemm, (hipStream_t)stream);
  const hipError_t err = mx::launch_gemm_quantize(p, (hipStream_t)stream);
  mx::profile_end(slot, (hipStream_t)stream);
  return err == hipSuccess ? MX_OK : MX_E_DEVICE;
}

mx_status mx_attn_fwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq, void* o, float* lse,
                      void* stream) {
  return fwd_impl(desc, nullptr, q_row, k_row, v_seq, o, lse, stream, false);
}

mx_status mx_attn_varlen_fwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq, void* o,
                             float* lse, void* stream) {
  return fwd_impl(desc, nullptr, q_row, k_row, v_seq, o, lse, stream, true);
}

mx_status mx_attn_fwd_strict(const mx_attn_desc* desc, mx_qview q_row, mx_qview k_row, mx_qview v_seq,
                             mx_qview v_tok, void* o, float* lse, void* stream) {
  return fwd_impl(desc, nullptr, q_row, k_row, v_seq, o, lse, stream, false, &v_tok);
}

mx_status mx_attn_cross_fwd(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview k_row,
                            mx_qview v_seq, void* o, float* lse, void* stream) {
  if (!seq_k) return MX_E_ARG;
  return fwd_impl(desc, seq_k, q_row, k_row, v_seq, o, lse, stream, false);
}

mx_status mx_attn_bwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row, mx_qview k_seq,
                      mx_qview v_row, const void* o, const float* lse, const void* g, mx_dtype g_dtype, void* dq,
                      void* dk, void* dv, void* stream) {
  return bwd_impl(desc, nullptr, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, false);
}

mx_status mx_attn_bwd_strict(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                             mx_qview k_seq, mx_qview k_tok, mx_qview v_row, const void* o, const float* lse,
                             const void* g, mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream) {
  return bwd_impl(desc, nullptr, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, false,
                  nullptr, &k_tok);
}

mx_status mx_attn_varlen_bwd(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                             mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* g,
                             mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream) {
  return bwd_impl(desc, nullptr, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, true);
}

mx_status mx_attn_bwd_noalloc(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row,
                              mx_qview k_seq, mx_qview v_row, const void* o, const float* lse, const void* g,
                              mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream) {
  mx::Geom geo, gk;
  mx_status st = check_desc(desc, &geo);
  if (st != MX_OK) return st;
  if (score_fp4(desc)) return MX_E_UNSUPPORTED;   // needs the dS code store, which the scratch lacks
  gk = geo;
  // the minimal workspace of this call must fit the scratch (checked before any device call)
  const size_t need = bwd_layout(geo, gk, desc).total;
  if (need > (size_t)MX_NOALLOC_SCRATCH_BYTES) return MX_E_WORKSPACE;
  void* ws = nullptr;
  if ((st = current_scratch(&ws)) != MX_OK) return st;
  mx_attn_desc d = *desc;
  d.workspace = ws;
  d.workspace_bytes = need;   // exactly the minimum: dQ rebuilds dS (no dS code store)
  return bwd_impl(&d, nullptr, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, false);
}

mx_status mx_attn_bwd_mx(const mx_attn_desc* desc, mx_qview q_row, mx_qview q_seq, mx_qview k_row, mx_qview k_seq,
                         mx_qview v_row, const void* o, const float* lse, const void* g, mx_dtype g_dtype, void* dq,
                         void* dk, void* dv, const mx_qview* dk_row, const mx_qview* dk_seq, const mx_qview* dv_row,
                         const mx_qview* dv_seq, void* stream) {
  const mx_qview none = {nullptr, nullptr};
  const mx_qview out[4] = {dk_row ? *dk_row : none, dk_seq ? *dk_seq : none, dv_row ? *dv_row : none,
                           dv_seq ? *dv_seq : none};
  return bwd_impl(desc, nullptr, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, false,
                  out);
}

mx_status mx_attn_cross_bwd(const mx_attn_desc* desc, const mx_seq* seq_k, mx_qview q_row, mx_qview q_seq,
                            mx_qview k_row, mx_qview k_seq, mx_qview v_row, const void* o, const float* lse,
                            const void* g, mx_dtype g_dtype, void* dq, void* dk, void* dv, void* stream) {
  if (!seq_k) return MX_E_ARG;
  return bwd_impl(desc, seq_k, q_row, q_seq, k_row, k_seq, v_row, o, lse, g, g_dtype, dq, dk, dv, stream, false);
}

size_t mx_attn_cross_workspace_size(const mx_attn_desc* desc, const mx_seq* seq_k, int32_t for_bwd) {
  mx::Geom g, gk;
  if (for_bwd != 1 && for_bwd != 2) return 0;
  if (!desc || !make_geom(&desc->seq, &g) || desc->heads_q < 1 || !valid_dim(desc->head_dim)) return 0;
  if (key_geom(desc, g, seq_k, &gk) != MX_OK) return 0;
  const BwdWorkspace w = bwd_layout(g, gk, desc);
  if (score_fp4(desc)) return w.store_ok ? w.total_store : 0;   // the store is required
  return for_bwd == 2 ? w.total_store : w.total;
}

size_t mx_attn_workspace_size(const mx_attn_desc* desc, int32_t for_bwd) {
  return mx_attn_cross_workspace_size(desc, nullptr, for_bwd);
}

size_t mx_view_codes_bytes(const mx_seq* seq, int32_t heads, int32_t head_dim, int32_t view) {
  mx::Geom g;
  if (!make_geom(seq, &g) || heads < 1 || !valid_dim(head_dim)) return 0;
  if (view == MX_VIEW_ROW) return row_codes_bytes(g, heads, head_dim);
  if (view == MX_VIEW_SEQ) return seq_codes_bytes(g, heads, head_dim);
  if (view == MX_VIEW_ROW_FP4) return row_codes_bytes(g, heads, head_dim) / 2;
  if (view == MX_VIEW_SEQ_TOKEN) return seq_codes_bytes(g, heads, head_dim);
  return 0;
}

size_t mx_view_scales_bytes(const mx_seq* seq, int32_t heads, int32_t head_dim, int32_t view) {
  // one scale byte per 32 elements in every view but the per-token one (one per token slot)
  if (view == MX_VIEW_SEQ_TOKEN) return valid_dim(head_dim) ? mx_view_codes_bytes(seq, heads, head_dim, view) / head_dim : 0;
  const int32_t elem_view = view == MX_VIEW_ROW_FP4 ? MX_VIEW_ROW : view;
  return mx_view_codes_bytes(seq, heads, head_dim, elem_view) / 32;
}

mx_status mx_read_flags(const void* workspace, uint32_t* flags) {
  if (!flags || !workspace) return MX_E_ARG;
  *flags = 0;
  return hipMemcpy(flags, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost) == hipSuccess ? MX_OK : MX_E_DEVICE;
}

mx_status mx_profile_kernel(int32_t kernel, void* const* start_events, void* const* stop_events, int32_t count) {
  mx::ProfileHook& h = mx::profile_hook();
  if (kernel == 0 || count <= 0) {
    h = mx::ProfileHook();
    return MX_OK;
  }
  if (kernel < 1 || kernel > 7 || !start_events || !stop_events) return MX_E_ARG;
  h.kind = kernel;
  h.start = (hipEvent_t*)start_events;
  h.stop = (hipEvent_t*)stop_events;
  h.n = count;
  h.count = 0;
  return MX_OK;
}

const char* mx_strerror(mx_status s) {
  switch (s) {
    case MX_OK: return "ok";
    case MX_E_ARG: return "invalid argument";
    case MX_E_UNSUPPORTED: return "unsupported configuration";
    case MX_E_WORKSPACE: return "workspace missing or too small";
    case MX_E_DEVICE: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t mx_abi_version(void) { return MXATTN_ABI_VERSION; }

}  // extern "C"
