// Host-side launchers of the verify-round kernels (defined in the .hip files).
#pragma once
#include <hip/hip_runtime.h>
#include "common.hpp"

namespace sv {

// projections
constexpr int kBarrierSpin = 1 << 21;   // default polls of one grid barrier (about a second)
int launch_proj(const ProjParams& p, bool swiglu, int xs, hipStream_t st);
// cut units of a balanced gate/up launch of N features over K (rem units of pq pieces
// each); returns rem * pq, 0 when the launch needs no cut
int swiglu_pieces(int N, int K, int* rem, int* pq);
int launch_gemm_f32(const GemmF32Params& p, bool swiglu, hipStream_t st);

// LM head statistics and the residual race
int lmhead_groups(int V, bool bf16);
int launch_lmhead(const LmParams& p, bool bf16, hipStream_t st);
int launch_race(const RaceParams& p, hipStream_t st);
// sampled rounds of a bf16 model: statistics, decisions and the residual race in one
// cooperative launch of `grid` workgroups (one per CU); -2 when the vocabulary is too
// large for the on-chip slices
int coop_grid();
int launch_lmhead_coop(const LmParams& p, int grid, hipStream_t st);

// fragment packing
int launch_pack_weight(const void* src, void* dst, int N, int K, hipStream_t st);
int launch_pack_rows(const void* src, void* dst, int R, int K, size_t plane, int xs, int* zero, int nzero,
                     hipStream_t st);

// attention
int launch_attention(const AttnParams& p, bool bf16, hipStream_t st);
int launch_attn_combine(const AttnParams& p, void* o, bool bf16, hipStream_t st);

// per-row layers
int launch_rope_table(const int32_t* kv_len, const RowInfo& ri, int d, float theta, double* table,
                      hipStream_t st);
int launch_embed_norm(const int32_t* tokens, const void* embed, int V, int H, const float* gain, float eps,
                      float* x, void* h, const RowInfo& ri, bool bf16, int* zero, int nzero, hipStream_t st);
int launch_resid_norm(const float* P, int S, float* x, int H, const float* gain, float eps, void* h,
                      const RowInfo& ri, bool bf16, hipStream_t st);
int launch_qkv_post(const float* P, int S, const double* rope, int use_rope, int nq, int nkv, int d,
                    float* q, void* sk, void* sv, const KvStage& ks, const RowInfo& ri, bool bf16, hipStream_t st);
int launch_gdn_verify(const float* P, int S, int hg, int dg, const float* state, int n_gdn, int gi,
                      float* stage, void* o, const RowInfo& ri, bool bf16, hipStream_t st);
int launch_gdn_replay(const int32_t* committed, float* state, int n_gdn, int hg, int dg, const float* stage,
                      size_t stage_layer_stride, const RowInfo& ri, hipStream_t st);
int launch_commit_kv(const int32_t* committed, const int32_t* kv_len, const int32_t* block_table, int max_blocks,
                     int n_blocks, void* kpool, void* vpool, int n_attn, int nkv, int d, const void* sk,
                     const void* sv, size_t stage_layer_elems, const RowInfo& ri, bool bf16, hipStream_t st);
int launch_kvlen_update(const int32_t* committed, int32_t* kv_len, const RowInfo& ri, hipStream_t st);
int launch_sum_partials(const float* P, int S, size_t n, float* Y, hipStream_t st);
int launch_copy_rows(const void* src, void* dst, size_t bytes, hipStream_t st);

// n-gram drafter and the history of a multi-round loop
int launch_ngram_draft(const int32_t* hist, const int32_t* hist_len, int lanes, int max_len, int k, int n_max,
                       int n_min, int32_t* tokens, int32_t* n_match, hipStream_t st);
int launch_counts_add(int32_t* counts, int vocab, int lanes, const int32_t* committed, const int32_t* out_tokens,
                      int out_stride, hipStream_t st);
int launch_history_append(int32_t* hist, int32_t* hist_len, int lanes, int max_len, const int32_t* committed,
                          const int32_t* out_tokens, int out_stride, hipStream_t st);

// acceptance
int launch_row_reduce(const LmPartial* part, int groups, int R, float inv_t, RowStat* rs, void* user_stats,
                      hipStream_t st);
int launch_lane_accept(const RowStat* rs, const int32_t* tokens, const int32_t* kv_len, const float* q, int V,
                       int sampled, float inv_t, uint32_t key0, uint32_t key1, LaneDecision* dec,
                       int32_t* committed, int32_t* out, const RowInfo& ri, hipStream_t st);
int launch_race_finish(const float* part, int groups, const LaneDecision* dec, int32_t* out,
                       const RowInfo& ri, hipStream_t st);
int launch_accept_coop(const RowStat* rs, const LaneDecision* dec, const float* part, const int* bar,
                       const int32_t* tokens, float inv_t, int32_t* committed, int32_t* out, void* user_stats,
                       const RowInfo& ri, hipStream_t st);

// the library's static device scratch on the current device (address and size); -1 on a
// HIP error
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
int static_scratch(void** ptr, size_t* bytes);

}  // namespace sv
