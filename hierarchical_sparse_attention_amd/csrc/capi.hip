// capi.hip - the extern "C" boundary of libhs_attn.so: host-side argument
// validation (before any HIP call), workspace layout and kernel dispatch.
// The declarations and their contracts are in include/hs_attn.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "hs_internal.h"

namespace {

using hs::KvView;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

hs_status check_kv(const hs_kv_cache* kv, bool need_k, bool need_v) {
  if (!kv) return HS_ERR_INVALID_ARG;
  if (kv->dtype != HS_F32 && kv->dtype != HS_BF16) return HS_ERR_UNSUPPORTED;
  if (kv->head_dim != 64 && kv->head_dim != 128) return HS_ERR_UNSUPPORTED;
  if (!kv->page_table || !kv->seq_lens) return HS_ERR_INVALID_ARG;
  if (kv->batch < 1 || kv->num_kv_heads < 1) return HS_ERR_INVALID_ARG;
  if ((int64_t)kv->batch * kv->num_kv_heads > 65535) return HS_ERR_UNSUPPORTED;
  if (kv->page_size < 1 || kv->max_pages < 1 || kv->num_phys_pages < 1) return HS_ERR_INVALID_ARG;
  if (kv->max_seq_len < 0 || (int64_t)kv->max_seq_len > (int64_t)kv->max_pages * kv->page_size)
    return HS_ERR_INVALID_ARG;
  if (need_k && (!kv->k_pool || !aligned16(kv->k_pool))) return HS_ERR_INVALID_ARG;
  if (need_v && (!kv->v_pool || !aligned16(kv->v_pool))) return HS_ERR_INVALID_ARG;
  return HS_OK;
}

KvView view_of(const hs_kv_cache* kv) {
  KvView v;
  v.k_pool = static_cast<const uint8_t*>(kv->k_pool);
  v.v_pool = static_cast<const uint8_t*>(kv->v_pool);
  v.page_table = kv->page_table;
  v.seq_lens = kv->seq_lens;
  v.batch = kv->batch;
  v.num_kv_heads = kv->num_kv_heads;
  v.head_dim = kv->head_dim;
  v.page_size = kv->page_size;
  v.max_pages = kv->max_pages;
  v.num_phys_pages = kv->num_phys_pages;
  v.max_seq_len = kv->max_seq_len;
  v.elem_bytes = kv->dtype == HS_BF16 ? 2 : 4;
  return v;
}

// blocks a level can have per unit
int64_t blocks_needed(const hs_kv_cache* kv, int32_t block_size) {
  return ceil_div(kv->max_seq_len, block_size);
}

hs_status check_summ(const hs_summaries* s, const hs_kv_cache* kv) {
  if (!s || !s->data || !aligned16(s->data)) return HS_ERR_INVALID_ARG;
  if (s->kind != HS_SUMMARY_MEAN && s->kind != HS_SUMMARY_MINMAX) return HS_ERR_INVALID_ARG;
  if (s->block_size < 1 || s->max_blocks < 1) return HS_ERR_INVALID_ARG;
  if (s->max_blocks > hs::kMaxBlocks) return HS_ERR_UNSUPPORTED;
  if ((int64_t)s->max_blocks < blocks_needed(kv, s->block_size)) return HS_ERR_INVALID_ARG;
  return HS_OK;
}

int group_size(const hs_kv_cache* kv, int32_t num_q_heads, hs_status* st) {
  *st = HS_OK;
  if (num_q_heads < 1 || num_q_heads % kv->num_kv_heads != 0) {
    *st = HS_ERR_INVALID_ARG;
    return 0;
  }
  const int G = num_q_heads / kv->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) *st = HS_ERR_UNSUPPORTED;
  return G;
}

// Workspace of hs_select_blocks (byte offsets).
// Workspace of hs_select_blocks: [arrival counters, 2 levels][coarse scores]
// [kept coarse ids][their counts][fine scores].
struct SelectLayout {
  bool two_level;
  int64_t units, nb_fine, nc, kc_cap, ratio, fine_slots;
  size_t off_cnt, off_coarse_scores, off_coarse_keys, off_gamma, off_gamma_cnt, off_fine_scores,
      off_fine_keys, total;
};

hs_status check_select(const hs_select_params* p, const hs_kv_cache* kv,
                       const hs_summaries* fine, const hs_summaries* coarse, SelectLayout* L) {
  if (!p) return HS_ERR_INVALID_ARG;
  hs_status st = check_kv(kv, false, false);
  if (st != HS_OK) return st;
  group_size(kv, p->num_q_heads, &st);
  if (st != HS_OK) return st;
  st = check_summ(fine, kv);
  if (st != HS_OK) return st;
  if (p->top_k < 0 || p->window_tokens < 0 || p->top_k_coarse < 0) return HS_ERR_INVALID_ARG;
  if (!(p->top_k_ratio >= 0.f && p->top_k_ratio <= 1.f)) return HS_ERR_INVALID_ARG;  // NaN too
  if (p->forced_cap < 0 || (p->forced_cap > 0) != (p->forced_ids != nullptr))
    return HS_ERR_INVALID_ARG;
  const bool two = p->top_k_coarse > 0;
  if (two) {
    st = check_summ(coarse, kv);
    if (st != HS_OK) return st;
    if (coarse->block_size % fine->block_size != 0) return HS_ERR_INVALID_ARG;
  }
  const int64_t S = fine->block_size;
  const int64_t nb = blocks_needed(kv, fine->block_size);
  const int64_t k = p->top_k_ratio > 0.f
                        ? std::max<int64_t>(1, (int64_t)((double)fine->max_blocks * (double)p->top_k_ratio))
                        : p->top_k;
  const int64_t need = std::min<int64_t>(
      fine->max_blocks,
      std::min<int64_t>(k, fine->max_blocks) + ceil_div(p->window_tokens, S) + 1 + p->forced_cap);
  if (p->max_selected < need || p->max_selected < 1) return HS_ERR_INVALID_ARG;

  L->two_level = two;
  L->units = (int64_t)kv->batch * kv->num_kv_heads;
  L->nb_fine = nb > 0 ? nb : 1;
  L->off_cnt = 0;  // fine level's counters, then the coarse level's
  size_t off = align_up(sizeof(int32_t) * hs::kCounterStride * 2 * L->units);
  if (two) {
    L->nc = std::max<int64_t>(1, blocks_needed(kv, coarse->block_size));
    L->kc_cap = std::min<int64_t>(p->top_k_coarse, L->nc);
    L->ratio = coarse->block_size / fine->block_size;
    L->fine_slots = std::max<int64_t>(1, L->kc_cap * L->ratio);
    L->off_coarse_scores = off;
    off = align_up(off + sizeof(float) * L->units * L->nc);
    L->off_coarse_keys = off;
    off = align_up(off + sizeof(uint32_t) * 2 * L->units * hs::step_chunks((int32_t)L->nc));
    L->off_gamma = off;
    off = align_up(off + sizeof(int32_t) * L->units * L->kc_cap);
    L->off_gamma_cnt = off;
    off = align_up(off + sizeof(int32_t) * L->units);
  } else {
    L->nc = L->kc_cap = 0;
    L->ratio = 1;
    L->fine_slots = L->nb_fine;
    L->off_coarse_scores = L->off_coarse_keys = L->off_gamma = L->off_gamma_cnt = 0;
  }
  L->off_fine_scores = off;
  off = align_up(off + sizeof(float) * L->units * L->fine_slots);
  L->off_fine_keys = off;
  off = align_up(off + sizeof(uint32_t) * 2 * L->units * hs::step_chunks((int32_t)L->fine_slots));
  L->total = off;
  return HS_OK;
}

// Workspace of hs_sparse_decode: [arrival counters][split partials o][(m, l)].
struct DecodeLayout {
  int64_t units, n_splits, G;
  size_t off_cnt, off_o, off_ml, total;
};

hs_status check_decode(const hs_kv_cache* kv, int32_t num_q_heads, int32_t block_size,
                       int32_t max_selected, DecodeLayout* L) {
  hs_status st = check_kv(kv, true, true);
  if (st != HS_OK) return st;
  const int G = group_size(kv, num_q_heads, &st);
  if (st != HS_OK) return st;
  if (block_size < 1 || max_selected < 1) return HS_ERR_INVALID_ARG;
  L->units = (int64_t)kv->batch * kv->num_kv_heads;
  L->G = G;
  L->n_splits = hs::decode_splits(L->units, max_selected, block_size);
  L->off_cnt = 0;
  L->off_o = align_up(sizeof(int32_t) * hs::kCounterStride * L->units);
  L->off_ml = align_up(L->off_o + sizeof(float) * L->units * L->n_splits * G * kv->head_dim);
  L->total = align_up(L->off_ml + sizeof(float) * L->units * L->n_splits * G * 2);
  return HS_OK;
}

hs_status from_hip(hipError_t e) { return e == hipSuccess ? HS_OK : HS_ERR_HIP; }

// The separate decode launch keeps each split task's run of the list in LDS.
hs_status check_decode_run(const hs_kv_cache* kv, int32_t block_size, int32_t max_selected,
                           const DecodeLayout& L) {
  const size_t run = hs::decode_run_bytes(kv->dtype == HS_BF16 ? 2 : 4, block_size, max_selected,
                                          (int)L.n_splits);
  return run <= hs::kDecodeRunLds ? HS_OK : HS_ERR_INVALID_ARG;
}

// Workspace of hs_select_decode: [control words][selection workspace][decode
// workspace].
struct StepLayout {
  SelectLayout sel;
  DecodeLayout dec;
  size_t off_ctrl, off_sel, off_dec, total;
};

hs_status check_step(const hs_select_params* p, const hs_kv_cache* kv, const hs_summaries* fine,
                     const hs_summaries* coarse, StepLayout* L) {
  hs_status st = check_select(p, kv, fine, coarse, &L->sel);
  if (st != HS_OK) return st;
  st = check_decode(kv, p->num_q_heads, fine->block_size, p->max_selected, &L->dec);
  if (st != HS_OK) return st;
  const int64_t chunks = hs::step_chunks((int32_t)L->sel.fine_slots);
  if (L->sel.units * (chunks + L->dec.n_splits) > 0x7FFFFFFF) return HS_ERR_UNSUPPORTED;
  L->off_ctrl = 0;
  L->off_sel = align_up(hs::kCtrlBytes);
  L->off_dec = align_up(L->off_sel + L->sel.total);
  L->total = align_up(L->off_dec + L->dec.total);
  return HS_OK;
}

// Selection parameters of the last level (the only one, or the fine level
// of two); a two-level selection first launches its coarse level on s, or,
// with coarse_out, only returns that level's parameters there.
hs_status select_params(const hs_select_params* prm, const hs_kv_cache* kv, const void* q,
                        const hs_summaries* fine, const hs_summaries* coarse,
                        int32_t* block_ids, int32_t* num_selected, uint8_t* ws,
                        const SelectLayout& L, hipStream_t s, hs::SelectParams* out,
                        hs::SelectParams* coarse_out = nullptr) {
  int32_t* counters = reinterpret_cast<int32_t*>(ws + L.off_cnt);
  hs::SelectParams sp;
  sp.kv = view_of(kv);
  sp.q = q;
  sp.G = prm->num_q_heads / kv->num_kv_heads;
  int32_t* gamma = nullptr;
  int32_t* gamma_cnt = nullptr;
  if (L.two_level) {
    gamma = reinterpret_cast<int32_t*>(ws + L.off_gamma);
    gamma_cnt = reinterpret_cast<int32_t*>(ws + L.off_gamma_cnt);
    sp.summ = coarse->data;
    sp.kind = coarse->kind;
    sp.block_size = coarse->block_size;
    sp.max_blocks = coarse->max_blocks;
    sp.gamma = nullptr;
    sp.gamma_cnt = nullptr;
    sp.gamma_cap = 0;
    sp.ratio = 1;
    sp.n_slots_max = (int32_t)L.nc;
    sp.scores = reinterpret_cast<float*>(ws + L.off_coarse_scores);
    sp.chunk_keys = reinterpret_cast<uint32_t*>(ws + L.off_coarse_keys);
    sp.top_k = prm->top_k_coarse;
    sp.top_k_ratio = 0.f;
    sp.forced = nullptr;
    sp.forced_cap = 0;
    sp.window = 0;
    sp.out_ids = gamma;
    sp.out_cnt = gamma_cnt;
    sp.out_cap = (int32_t)L.kc_cap;
    sp.out_blocks_max = (int32_t)L.nc;
    sp.counters = counters + L.units * hs::kCounterStride;
    sp.refresh_begin = -1;
    if (coarse_out) {
      *coarse_out = sp;
    } else {
      const hipError_t e = hs::launch_select(sp, s);
      if (e != hipSuccess) return from_hip(e);
    }
  }
  sp.summ = fine->data;
  sp.kind = fine->kind;
  sp.block_size = fine->block_size;
  sp.max_blocks = fine->max_blocks;
  sp.gamma = gamma;
  sp.gamma_cnt = gamma_cnt;
  sp.gamma_cap = (int32_t)L.kc_cap;
  sp.ratio = (int32_t)L.ratio;
  sp.n_slots_max = (int32_t)L.fine_slots;
  sp.scores = reinterpret_cast<float*>(ws + L.off_fine_scores);
  sp.chunk_keys = reinterpret_cast<uint32_t*>(ws + L.off_fine_keys);
  sp.top_k = prm->top_k;
  sp.top_k_ratio = prm->top_k_ratio;
  sp.forced = prm->forced_ids;
  sp.forced_cap = prm->forced_cap;
  sp.window = prm->window_tokens;
  sp.out_ids = block_ids;
  sp.out_cnt = num_selected;
  sp.out_cap = prm->max_selected;
  sp.out_blocks_max = (int32_t)L.nb_fine;
  sp.counters = counters;
  sp.refresh_begin = -1;
  *out = sp;
  return HS_OK;
}

hs::DecodeParams decode_params(const hs_kv_cache* kv, const void* q, float scale,
                               int32_t block_size, const int32_t* block_ids,
                               const int32_t* num_selected, int32_t max_selected, float* out,
                               uint8_t* ws, const DecodeLayout& L) {
  if (scale == 0.f) scale = 1.0f / sqrtf((float)kv->head_dim);
  hs::DecodeParams p;
  p.kv = view_of(kv);
  p.q = q;
  p.G = (int32_t)L.G;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.block_size = block_size;
  p.ids = block_ids;
  p.counts = num_selected;
  p.max_selected = max_selected;
  p.n_splits = (int32_t)L.n_splits;
  p.part_o = reinterpret_cast<float*>(ws + L.off_o);
  p.part_ml = reinterpret_cast<float*>(ws + L.off_ml);
  p.counters = reinterpret_cast<int32_t*>(ws + L.off_cnt);
  p.score_counters = nullptr;
  p.score_chunks = 0;
  p.out = out;
  return p;
}

// Token-level second stage: workspace [counters][scores][chunk key ranges]
// and the level's parameters.
struct TokenLayout {
  int64_t units, n_slots;
  size_t off_cnt, off_scores, off_keys, total;
};

hs_status check_tokens(const hs_kv_cache* kv, int32_t num_q_heads, int32_t block_size,
                       int32_t max_selected, int32_t top_k_tokens, int32_t window_tokens,
                       int32_t max_tokens, TokenLayout* L) {
  hs_status st = check_kv(kv, true, false);
  if (st != HS_OK) return st;
  group_size(kv, num_q_heads, &st);
  if (st != HS_OK) return st;
  if (block_size < 1 || max_selected < 1 || top_k_tokens < 0 || window_tokens < 0 ||
      max_tokens < 1)
    return HS_ERR_INVALID_ARG;
  const int64_t n_slots = (int64_t)max_selected * block_size;
  if (n_slots > (1 << 24)) return HS_ERR_UNSUPPORTED;
  const int64_t need = std::min<int64_t>(n_slots, top_k_tokens) +
                       std::min<int64_t>(window_tokens, kv->max_seq_len);
  if (max_tokens < need) return HS_ERR_INVALID_ARG;
  if (!hs::tokens_in_registers(hs::kKindTokens, (int32_t)n_slots, max_selected) &&
      hs::select_launch_lds_bytes(kv->max_seq_len, (int32_t)n_slots, max_tokens) >
          (size_t)HS_TOKEN_LDS_BYTES)
    return HS_ERR_UNSUPPORTED;
  L->units = (int64_t)kv->batch * kv->num_kv_heads;
  L->n_slots = n_slots;
  L->off_cnt = 0;
  L->off_scores = align_up(sizeof(int32_t) * hs::kCounterStride * L->units);
  L->off_keys = align_up(L->off_scores + sizeof(float) * L->units * n_slots);
  L->total = align_up(L->off_keys + sizeof(uint32_t) * 2 * L->units *
                                         hs::step_chunks((int32_t)n_slots));
  return HS_OK;
}

}  // namespace

extern "C" {

hs_status hs_select_tokens_workspace_size(const hs_kv_cache* kv, int32_t num_q_heads,
                                          int32_t block_size, int32_t max_selected,
                                          int32_t top_k_tokens, int32_t window_tokens,
                                          int32_t max_tokens, size_t* bytes) {
  if (!bytes) return HS_ERR_INVALID_ARG;
  TokenLayout L;
  const hs_status st = check_tokens(kv, num_q_heads, block_size, max_selected, top_k_tokens,
                                    window_tokens, max_tokens, &L);
  if (st == HS_OK) *bytes = L.total;
  return st;
}

hs_status hs_select_tokens(const hs_kv_cache* kv, const void* q, int32_t num_q_heads,
                           int32_t block_size, const int32_t* block_ids,
                           const int32_t* num_selected, int32_t max_selected,
                           int32_t top_k_tokens, int32_t window_tokens, int32_t* token_ids,
                           int32_t* num_tokens, int32_t max_tokens, void* workspace,
                           size_t workspace_bytes, void* stream) {
  TokenLayout L;
  hs_status st = check_tokens(kv, num_q_heads, block_size, max_selected, top_k_tokens,
                              window_tokens, max_tokens, &L);
  if (st != HS_OK) return st;
  if (!q || !aligned16(q) || !block_ids || !num_selected || !token_ids || !num_tokens)
    return HS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return HS_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hs::SelectParams sp;
  sp.kv = view_of(kv);
  sp.q = q;
  sp.summ = nullptr;
  sp.kind = hs::kKindTokens;
  sp.block_size = 1;  // a candidate is one token
  sp.max_blocks = kv->max_seq_len;
  sp.G = num_q_heads / kv->num_kv_heads;
  sp.gamma = block_ids;  // the selected blocks play the coarse level: slot c is token
  sp.gamma_cnt = num_selected;  // block_ids[c / S] * S + c % S
  sp.gamma_cap = max_selected;
  sp.ratio = block_size;
  sp.n_slots_max = (int32_t)L.n_slots;
  sp.scores = reinterpret_cast<float*>(ws + L.off_scores);
  sp.chunk_keys = reinterpret_cast<uint32_t*>(ws + L.off_keys);
  sp.top_k = top_k_tokens;
  sp.top_k_ratio = 0.f;
  sp.forced = nullptr;
  sp.forced_cap = 0;
  sp.window = window_tokens;
  sp.out_ids = token_ids;
  sp.out_cnt = num_tokens;
  sp.out_cap = max_tokens;
  sp.out_blocks_max = kv->max_seq_len;
  sp.counters = reinterpret_cast<int32_t*>(ws + L.off_cnt);
  sp.refresh_begin = -1;
  return from_hip(hs::launch_select(sp, static_cast<hipStream_t>(stream)));
}


const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "HS_OK";
    case HS_ERR_INVALID_ARG: return "HS_ERR_INVALID_ARG";
    case HS_ERR_UNSUPPORTED: return "HS_ERR_UNSUPPORTED";
    case HS_ERR_WORKSPACE: return "HS_ERR_WORKSPACE";
    case HS_ERR_HIP: return "HS_ERR_HIP";
  }
  return "HS_UNKNOWN_STATUS";
}

int32_t hs_version(void) { return HS_ATTN_VERSION; }

hs_status hs_select_workspace_size(const hs_select_params* p, const hs_kv_cache* kv,
                                   const hs_summaries* fine, const hs_summaries* coarse,
                                   size_t* bytes) {
  if (!bytes) return HS_ERR_INVALID_ARG;
  SelectLayout L;
  const hs_status st = check_select(p, kv, fine, coarse, &L);
  if (st == HS_OK) *bytes = L.total;
  return st;
}

hs_status hs_decode_workspace_size(const hs_kv_cache* kv, int32_t num_q_heads,
                                   int32_t block_size, int32_t max_selected, size_t* bytes) {
  if (!bytes) return HS_ERR_INVALID_ARG;
  DecodeLayout L;
  hs_status st = check_decode(kv, num_q_heads, block_size, max_selected, &L);
  if (st == HS_OK) st = check_decode_run(kv, block_size, max_selected, L);
  if (st == HS_OK) *bytes = L.total;
  return st;
}

hs_status hs_build_summaries(const hs_kv_cache* kv, int32_t block_begin, const hs_summaries* out,
                             void* stream) {
  hs_status st = check_kv(kv, true, false);
  if (st != HS_OK) return st;
  st = check_summ(out, kv);
  if (st != HS_OK) return st;
  if (block_begin < 0) return HS_ERR_INVALID_ARG;
  hs::SummParams p;
  p.kv = view_of(kv);
  p.out = out->data;
  p.kind = out->kind;
  p.block_size = out->block_size;
  p.max_blocks = out->max_blocks;
  p.block_begin = block_begin;
  return from_hip(hs::launch_build_summaries(p, static_cast<hipStream_t>(stream)));
}

hs_status hs_append_kv(const hs_kv_cache* kv, const void* k_new, const void* v_new,
                       int32_t* seq_lens, void* stream) {
  const hs_status st = check_kv(kv, true, true);
  if (st != HS_OK) return st;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return HS_ERR_INVALID_ARG;
  if (!seq_lens || seq_lens != kv->seq_lens) return HS_ERR_INVALID_ARG;
  hs::AppendParams p;
  p.kv = view_of(kv);
  p.k_pool = static_cast<uint8_t*>(const_cast<void*>(kv->k_pool));
  p.v_pool = static_cast<uint8_t*>(const_cast<void*>(kv->v_pool));
  p.k_new = k_new;
  p.v_new = v_new;
  p.seq_lens = seq_lens;
  return from_hip(hs::launch_append(p, static_cast<hipStream_t>(stream)));
}

hs_status hs_block_cache_update(const hs_block_cache* cache, int32_t units, int32_t step,
                                const int32_t* block_ids, const int32_t* num_selected,
                                int32_t max_selected, int32_t* slot_of, int32_t* miss_blocks,
                                int32_t* stats, void* stream) {
  if (!cache || !cache->slot_block || !cache->slot_stamp) return HS_ERR_INVALID_ARG;
  if (!block_ids || !num_selected || !slot_of || !miss_blocks || !stats) return HS_ERR_INVALID_ARG;
  if (units < 1 || units > 65535 || step < 0 || step == 0x7FFFFFFF) return HS_ERR_INVALID_ARG;
  if (max_selected < 1 || cache->capacity < max_selected) return HS_ERR_INVALID_ARG;
  if (max_selected > hs::kMaxCacheSelected || cache->capacity > hs::kMaxCacheSlots)
    return HS_ERR_UNSUPPORTED;
  hs::CacheParams p;
  p.slot_block = cache->slot_block;
  p.slot_stamp = cache->slot_stamp;
  p.capacity = cache->capacity;
  p.units = units;
  p.step = step;
  p.max_selected = max_selected;
  p.ids = block_ids;
  p.counts = num_selected;
  p.slot_of = slot_of;
  p.miss_blocks = miss_blocks;
  p.stats = stats;
  return from_hip(hs::launch_cache_update(p, static_cast<hipStream_t>(stream)));
}

hs_status hs_select_blocks(const hs_select_params* prm, const hs_kv_cache* kv, const void* q,
                           const hs_summaries* fine, const hs_summaries* coarse,
                           int32_t* block_ids, int32_t* num_selected, void* workspace,
                           size_t workspace_bytes, void* stream) {
  SelectLayout L;
  hs_status st = check_select(prm, kv, fine, coarse, &L);
  if (st != HS_OK) return st;
  if (!q || !aligned16(q) || !block_ids || !num_selected) return HS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return HS_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hs::SelectParams sp;
  st = select_params(prm, kv, q, fine, coarse, block_ids, num_selected,
                     static_cast<uint8_t*>(workspace), L, s, &sp);
  if (st != HS_OK) return st;
  return from_hip(hs::launch_select(sp, s));
}

hs_status hs_sparse_decode(const hs_kv_cache* kv, const void* q, int32_t num_q_heads, float scale,
                           int32_t block_size, const int32_t* block_ids,
                           const int32_t* num_selected, int32_t max_selected, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  DecodeLayout L;
  hs_status st = check_decode(kv, num_q_heads, block_size, max_selected, &L);
  if (st == HS_OK) st = check_decode_run(kv, block_size, max_selected, L);
  if (st != HS_OK) return st;
  if (!q || !aligned16(q) || !block_ids || !num_selected || !out) return HS_ERR_INVALID_ARG;
  if (!isfinite(scale)) return HS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return HS_ERR_WORKSPACE;
  const hs::DecodeParams p = decode_params(kv, q, scale, block_size, block_ids, num_selected,
                                           max_selected, out, static_cast<uint8_t*>(workspace), L);
  return from_hip(hs::launch_decode(p, static_cast<hipStream_t>(stream)));
}

hs_status hs_select_decode_workspace_size(const hs_select_params* p, const hs_kv_cache* kv,
                                          const hs_summaries* fine, const hs_summaries* coarse,
                                          size_t* bytes) {
  if (!bytes) return HS_ERR_INVALID_ARG;
  StepLayout L;
  const hs_status st = check_step(p, kv, fine, coarse, &L);
  if (st == HS_OK) *bytes = L.total;
  return st;
}

}  // extern "C"

namespace {

// hs_select_decode and hs_decode_step; refresh_begin < 0: no refresh.
hs_status select_decode(const hs_select_params* prm, const hs_kv_cache* kv, const void* q,
                        const hs_summaries* fine, const hs_summaries* coarse, int32_t refresh_begin,
                        float scale, int32_t* block_ids, int32_t* num_selected, float* out,
                        void* workspace, size_t workspace_bytes, hipStream_t s) {
  StepLayout L;
  hs_status st = check_step(prm, kv, fine, coarse, &L);
  if (st != HS_OK) return st;
  if (!q || !aligned16(q) || !block_ids || !num_selected || !out) return HS_ERR_INVALID_ARG;
  if (!isfinite(scale)) return HS_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return HS_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  hs::StepParams p;
  if (refresh_begin >= 0 && L.sel.two_level) {
    // two levels: both tables are refreshed before the coarse selection reads
    // the coarse one; where the shapes allow, refreshes and coarse selection
    // are one launch (the two-level head), else three
    const int32_t cb = (int32_t)((int64_t)refresh_begin * fine->block_size / coarse->block_size);
    hs::SelectParams cp;
    st = select_params(prm, kv, q, fine, coarse, block_ids, num_selected, ws + L.off_sel, L.sel,
                       s, &p.sel, &cp);
    if (st != HS_OK) return st;
    if (hs::two_level_head_fits(cp, fine->block_size, coarse->kind)) {
      hs::HeadParams h;
      h.fine = fine->data;
      h.fine_kind = fine->kind;
      h.fine_block = fine->block_size;
      h.fine_max_blocks = fine->max_blocks;
      h.fine_begin = refresh_begin;
      h.coarse_begin = cb;
      h.status = reinterpret_cast<int32_t*>(ws + L.off_ctrl) + hs::kCtrlStatus;
      const hipError_t e = hs::launch_two_level_head(cp, h, s);
      if (e != hipSuccess) return from_hip(e);
    } else {
      hs_status r = hs_build_summaries(kv, refresh_begin, fine, s);
      if (r != HS_OK) return r;
      r = hs_build_summaries(kv, cb, coarse, s);
      if (r != HS_OK) return r;
      const hipError_t e = hs::launch_select(cp, s);
      if (e != hipSuccess) return from_hip(e);
    }
    refresh_begin = -1;
  } else {
    st = select_params(prm, kv, q, fine, coarse, block_ids, num_selected, ws + L.off_sel, L.sel,
                       s, &p.sel);
    if (st != HS_OK) return st;
  }
  p.dec = decode_params(kv, q, scale, fine->block_size, block_ids, num_selected,
                        prm->max_selected, out, ws + L.off_dec, L.dec);
  p.sel.refresh_begin = refresh_begin;
  if (!hs::step_fits(p.sel.out_blocks_max, p.sel.n_slots_max, p.sel.out_cap) ||
      fine->block_size == 1) {
    // id lists too long for the fused kernel's LDS, or one-token blocks (the
    // token-list attention is compiled into the separate decode kernel only):
    // the stages as separate launches, with the same results
    if (refresh_begin >= 0) {
      const hs_status r = hs_build_summaries(kv, refresh_begin, fine, s);
      if (r != HS_OK) return r;
      p.sel.refresh_begin = -1;
    }
    const hipError_t e = hs::launch_select(p.sel, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(hs::launch_decode(p.dec, s));
  }
  p.units = (int32_t)L.sel.units;
  p.n_chunks = hs::step_chunks(p.sel.n_slots_max);
  p.total = p.units * (p.n_chunks + p.dec.n_splits);
  p.list_cap = p.sel.out_cap;
  p.dec.score_counters = p.sel.counters;
  p.dec.score_chunks = p.n_chunks;
  p.ctrl = reinterpret_cast<int32_t*>(ws + L.off_ctrl);
  p.wait_ticks = 0;  // set by launch_step from the device's wall-clock rate
  return from_hip(hs::launch_step(p, s));
}

}  // namespace

extern "C" {

hs_status hs_select_decode(const hs_select_params* prm, const hs_kv_cache* kv, const void* q,
                           const hs_summaries* fine, const hs_summaries* coarse, float scale,
                           int32_t* block_ids, int32_t* num_selected, float* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  return select_decode(prm, kv, q, fine, coarse, -1, scale, block_ids, num_selected, out,
                       workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

hs_status hs_step_status(const void* workspace, size_t workspace_bytes, int32_t* status,
                         void* stream) {
  if (!workspace || !status) return HS_ERR_INVALID_ARG;
  if (workspace_bytes < sizeof(int32_t)) return HS_ERR_WORKSPACE;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, static_cast<const int32_t*>(workspace) + hs::kCtrlStatus,
                                sizeof(v), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return HS_ERR_HIP;
  *status = v;
  return HS_OK;
}

hs_status hs_decode_step(const hs_select_params* prm, const hs_kv_cache* kv, const void* q,
                         const hs_summaries* fine, const hs_summaries* coarse,
                         int32_t refresh_begin, float scale, int32_t* block_ids,
                         int32_t* num_selected, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (refresh_begin < 0) return HS_ERR_INVALID_ARG;
  if (kv && (!kv->k_pool || !aligned16(kv->k_pool))) return HS_ERR_INVALID_ARG;
  return select_decode(prm, kv, q, fine, coarse, refresh_begin, scale, block_ids, num_selected,
                       out, workspace, workspace_bytes, static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ------------------------------------------------ no-allocation decode step
// hs_decode_step_noalloc runs hs_decode_step with its workspace in `scratch`,
// a device array of this library. Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress and kept in
// scratch_dev[]; every use goes through that address.
static __device__ __align__(256) uint8_t scratch[HS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];  // device address of `scratch` per device, once looked up

hs_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return HS_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return HS_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return HS_ERR_HIP;
    scratch_dev[dev] = p;
  }
  *out = scratch_dev[dev];
  return HS_OK;
}

// Zeroes [0, n0) and [off1, off1 + n1) bytes of `base` (multiples of 16): the
// control line and arrival counters that a call needs at zero. A kernel, not
// hipMemsetAsync, so that the call can be captured into a graph.
__global__ void k_clear_counters(uint8_t* base, int64_t n0, int64_t off1, int64_t n1) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x * 16;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 16; i < n0 + n1;
       i += stride) {
    const int64_t at = i < n0 ? i : off1 + (i - n0);
    *reinterpret_cast<uint4*>(base + at) = make_uint4(0, 0, 0, 0);
  }
}

}  // namespace

extern "C" {

hs_status hs_decode_step_noalloc(const hs_select_params* prm, const hs_kv_cache* kv,
                                 const void* q, const hs_summaries* fine,
                                 const hs_summaries* coarse, int32_t refresh_begin, float scale,
                                 int32_t* block_ids, int32_t* num_selected, float* out,
                                 void* stream) {
  // every argument is checked, and the size against the array's, before any HIP call
  if (refresh_begin < 0) return HS_ERR_INVALID_ARG;
  if (kv && (!kv->k_pool || !aligned16(kv->k_pool))) return HS_ERR_INVALID_ARG;
  StepLayout L;
  hs_status st = check_step(prm, kv, fine, coarse, &L);
  if (st != HS_OK) return st;
  if (!q || !aligned16(q) || !block_ids || !num_selected || !out) return HS_ERR_INVALID_ARG;
  if (!isfinite(scale)) return HS_ERR_INVALID_ARG;
  if (L.total > (size_t)HS_NOALLOC_SCRATCH_BYTES) return HS_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != HS_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  // the control line and the selection's counters are contiguous at the
  // start; the attention's counters start its part
  const int64_t n0 = (int64_t)(L.off_sel + align_up(sizeof(int32_t) * hs::kCounterStride * 2 *
                                                   L.sel.units));
  const int64_t n1 = (int64_t)align_up(sizeof(int32_t) * hs::kCounterStride * L.dec.units);
  hipLaunchKernelGGL(k_clear_counters, dim3(64), dim3(256), 0, s, static_cast<uint8_t*>(ws), n0,
                     (int64_t)L.off_dec, n1);
  if (hipGetLastError() != hipSuccess) return HS_ERR_HIP;
  return select_decode(prm, kv, q, fine, coarse, refresh_begin, scale, block_ids, num_selected,
                       out, ws, (size_t)HS_NOALLOC_SCRATCH_BYTES, s);
}

}  // extern "C"
