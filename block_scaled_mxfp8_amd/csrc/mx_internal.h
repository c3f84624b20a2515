// Internal launcher interface between the C ABI (mxattn_api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_layout.h"

namespace mx {

struct QuantizeParams {
  Geom geom;
  int heads;
  int head_dim;
  bool f32;              // input dtype: fp32 (else bf16)
  bool token_block;      // one exponent per 32-token block x all channels (else per-axis groups)
  const void* x;
  uint8_t* row_codes;    // nullptr: ROW view not wanted
  uint8_t* row_scales;
  bool row_fp4;          // the ROW view in MXFP4 (E2M1 codes, two per byte) instead of E4M3
  uint8_t* seq_codes;    // nullptr: SEQ view not wanted
  uint8_t* seq_scales;
  bool seq_token;        // the SEQ codes with one exponent per token (all channels); seq_scales
                         // then holds one byte per token, [group row][32]
  // backward preprocessing (all nullptr for a plain quantise): with `o` set, the kernel also
  // writes ndelta[token, head] = -sum_c dequant(ROW code) * O (that is -D) and
  // lse2[token, head] = lse * log2 e, the forms the backward kernels consume.
  const void* o;
  bool o_f32;
  float* ndelta;
  const float* lse;
  float* lse2;
  float* gnorm;          // nullptr, or |G~_row|_2 per (token, head) (the prefix dQ boost)
};

struct AttnParams {
  Geom geom;             // queries (and O, LSE)
  Geom geom_k;           // keys and values: the same as geom for self-attention
  int heads_q, heads_kv, head_dim;
  int causal;
  float scale;           // alpha
  bool out_f32;          // O / dQ / dK / dV storage type (else bf16)
  int plan;              // packed: 1D grid over the device-built work list (mx_worklist.h)
  bool score_fp4;        // Q and K ROW views are MXFP4 (E2M1 codes, d/2 bytes per token)
  // forward operands
  const uint8_t* q_codes; const uint8_t* q_scales;    // ROW view of Q
  const uint8_t* k_codes; const uint8_t* k_scales;    // ROW view of K
  const uint8_t* v_codes; const uint8_t* v_scales;    // SEQ view of V
  // strict per-key V fold (causal): the per-token view of V (SEQ code layout, one scale byte per
  // token); nullptr: the plain forward
  const uint8_t* vt_codes; const uint8_t* vt_scales;
  void* o;
  float* lse;
};

struct BwdParams {
  Geom geom;             // queries (and G, O, LSE, dQ)
  Geom geom_k;           // keys and values (and dK, dV): the same as geom for self-attention
  int heads_q, heads_kv, head_dim;
  int causal;
  float scale;
  bool out_f32;
  int plan;              // packed: 1D grids over the device-built work lists (mx_worklist.h)
  bool score_fp4;        // Q and K ROW views (the score operands) are MXFP4; needs the dS store
  int dq_mode;
  const uint8_t* q_codes; const uint8_t* q_scales;      // ROW Q
  const uint8_t* qs_codes; const uint8_t* qs_scales;    // SEQ Q
  const uint8_t* k_codes; const uint8_t* k_scales;      // ROW K
  const uint8_t* ks_codes; const uint8_t* ks_scales;    // SEQ K
  const uint8_t* vr_codes; const uint8_t* vr_scales;    // ROW V
  // strict dQ (causal, FP32 dQ): the per-token view of K (SEQ code layout, one scale byte per
  // token); nullptr: the plain backward
  const uint8_t* kt_codes; const uint8_t* kt_scales;
  const void* o;
  const float* lse;
  const void* g;
  bool g_f32;
  void* dq; void* dk; void* dv;
  // workspace pieces
  uint8_t* gr_codes; uint8_t* gr_scales;                // ROW G
  uint8_t* gs_codes; uint8_t* gs_scales;                // SEQ G
  float* ndelta;                                        // -D per (row, head)
  float* lse2;                                          // LSE * log2 e per (row, head)
  uint32_t* flags;
  // prefix dQ boost (dq_mode 2): |G~_row| per (row, head); prefix maxima of |V~_row,j|_2 and of
  // max_c |K~_seq,jc| per (key, KV head)
  float* gnorm; float* vpre; float* kpre;
  // dS code store (nullptr: dQ recomputes dS instead); layout in mx_layout.h DsStore
  uint8_t* ds_codes; uint8_t* ds_exps;
  DsStore ds;
  // optional MX views of dK and dV (the keys' geometry, layouts of mx_quantize), formed from
  // the FP32 accumulators; all nullptr: none
  uint8_t* dkr_codes; uint8_t* dkr_scales; uint8_t* dks_codes; uint8_t* dks_scales;
  uint8_t* dvr_codes; uint8_t* dvr_scales; uint8_t* dvs_codes; uint8_t* dvs_scales;
};

hipError_t launch_quantize(const QuantizeParams& p, hipStream_t stream);
hipError_t launch_attn_fwd(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream);

}  // namespace mx
