// C ABI of the verify round: validation, the row-budget planner, workspace
// layout and the launch sequence on the caller's stream.  No device memory is
// allocated here; the caller owns every device buffer.
#include "spec_verify.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "common.hpp"
#include "launch.hpp"

static_assert(sizeof(spec_row_stat) == sizeof(sv::spec_row_stat_dev), "row stat mirror");
static_assert(sizeof(sv::LmPartial) == 32, "partial size");

namespace {

constexpr int kDefaultChunk = 512;
constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layer {
  int kind;
  spec_layer_weights w;
  int attn_index;   // index among attention layers, or -1
  int gdn_index;    // index among gated-delta-rule layers, or -1
};

// K split of one projection: a function of (N, K) only, so results never depend on R.
struct Split {
  int S;
};

}  // namespace

struct spec_model {
  spec_model_desc d;
  std::vector<int32_t> kinds;
  std::vector<Layer> layers;
  int n_attn = 0, n_gdn = 0;
  bool bf16 = false;
  int chunk = kDefaultChunk;
  Split s_in_attn{1}, s_in_gdn{1}, s_o_attn{1}, s_o_gdn{1}, s_gateup{1}, s_down{1};
  int lm_groups = 1;
  int barrier_spin = sv::kBarrierSpin;   // polls per grid barrier of the cooperative head
  // profiling
  int prof_class = SPEC_K_NONE;
  int prof_every = 1;             // record launches 0, every, 2 every, ... of the class
  long prof_seen = 0;             // launches of the class since the last enable
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_events;
  std::vector<hipEvent_t> prof_pool;
  size_t prof_used = 0;
};

namespace {

// K splits of a bf16 projection, a function of (N, K) only so that results never
// depend on R: the largest S (at most `cap`, with at least two 256-wide units per split)
// for which the tiles of all splits fit eight to a workgroup of the one-per-CU launch.
// Eight tiles keep one weight-streaming wave per SIMD; a fifth tile pair would share a
// SIMD with another MFMA-heavy wave, and the younger of the two is starved of MFMA issue
// until the older one ends.  The input projections are capped at four splits: the
// attention prologue and the recurrent verify load four splits of their inputs in one
// batch, and a fifth costs another memory round trip.  The gate/up pair is never split
// (its SwiGLU epilogue needs the full sums).
int split_for(const spec_model* m, int N, int K, bool fused_pair, int cap = 8) {
  if (!m->bf16 || fused_pair) return 1;
  const int tiles = (N + 15) / 16;
  const int units = K / 256;
  int S = 1;
  while (S < cap && 2 * (S + 1) <= units && tiles * (S + 1) <= 8 * sv::kCUs) ++S;
  return S;
}

struct WsLayout {
  size_t x, h, P, q, o, a, pieces, pcnt, bar, rope, stk, stv, gst, apart, lmp, rstat, dec, racep, total;
  int n_cnt;                    // counters zeroed at the start of a round: the gate/up cut units', then the
                                // sampled head's grid barrier (kCoopCounters)
  size_t stage_layer_elems;     // elements per attention layer in stk/stv
  size_t gst_layer_floats;      // floats per gdn layer in gst
  int n_chunks;
};

size_t act_bytes(const spec_model* m) { return m->bf16 ? 2 : 4; }

WsLayout layout(const spec_model* m, int R, int L, int max_blocks) {
  const spec_model_desc& d = m->d;
  const size_t ab = act_bytes(m);
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max<size_t>(bytes, 1)); return o; };
  const size_t H = d.hidden;
  const size_t qdim = (size_t)d.n_q_heads * d.head_dim;
  const size_t gdim = (size_t)d.gdn_heads * d.gdn_dim;
  size_t pmax = 0;   // max S * N over partial-producing projections
  if (m->n_attn) {
    pmax = std::max(pmax, (size_t)m->s_in_attn.S * (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim);
    pmax = std::max(pmax, (size_t)m->s_o_attn.S * H);
  }
  if (m->n_gdn) {
    pmax = std::max(pmax, (size_t)m->s_in_gdn.S * (3 * gdim + 2 * d.gdn_heads));
    pmax = std::max(pmax, (size_t)m->s_o_gdn.S * H);
  }
  if (d.n_layers) pmax = std::max(pmax, (size_t)m->s_down.S * H);
  // activations are float32: an fp32 model keeps them as floats [R][width], a
  // bf16 model as hi/lo bf16 planes in fragment order, 16 ceil(R / 16) rows each
  // (the same four bytes per element)
  const size_t R16 = (size_t)sv::round16(R);
  w.x = take((size_t)R * H * 4);
  w.h = take(R16 * H * 4);
  w.P = take((size_t)R * pmax * 4);
  w.q = take((size_t)R * qdim * 4);
  w.o = take(R16 * std::max(qdim, gdim) * 4);
  w.a = take(R16 * d.ffn * 4);
  int rem = 0, pq = 0;
  if (m->bf16 && d.n_layers) sv::swiglu_pieces(d.ffn, (int)H, &rem, &pq);
  w.n_cnt = rem + sv::kCoopCounters;
  w.pieces = take((size_t)rem * pq * 2 * R * 16 * 4);
  w.pcnt = take((size_t)w.n_cnt * 4);
  w.bar = w.pcnt + (size_t)rem * 4;
  w.rope = take((size_t)R * (d.head_dim / 2) * 2 * 8);
  w.stage_layer_elems = (size_t)L * sv::kStageBlocks * SPEC_KV_BLOCK * d.n_kv_heads * d.head_dim;
  w.stk = take((size_t)m->n_attn * w.stage_layer_elems * ab);
  w.stv = take((size_t)m->n_attn * w.stage_layer_elems * ab);
  w.gst_layer_floats = (size_t)R * d.gdn_heads * (2 * 128 + 2);
  w.gst = take((size_t)m->n_gdn * w.gst_layer_floats * 4);
  w.n_chunks = m->n_attn ? (max_blocks * SPEC_KV_BLOCK + m->chunk - 1) / m->chunk : 0;
  w.apart = take((size_t)L * d.n_kv_heads * w.n_chunks * 64 * (d.head_dim + sv::kAttnPartPad) * 4);
  // partials per row (LM head) and per lane (residual race): one per group of the greedy
  // head or per workgroup of the sampled bf16 head's cooperative launch (at most kCUs)
  const size_t groups = (size_t)std::max(m->lm_groups, m->bf16 ? sv::kCUs : 0);
  w.lmp = take((size_t)R * groups * sizeof(sv::LmPartial));
  w.rstat = take((size_t)R * sizeof(sv::RowStat));
  w.dec = take((size_t)L * sizeof(sv::LaneDecision));
  w.racep = take((size_t)L * groups * 16);
  w.total = off;
  return w;
}

// The buffers of a head-only round (spec_verify_head, then spec_accept) alone: the hidden
// rows, the counters, the LM-head and race partials, the row statistics and decisions.
WsLayout head_layout(const spec_model* m, int R, int L) {
  const spec_model_desc& d = m->d;
  WsLayout w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + std::max<size_t>(bytes, 1)); return o; };
  w.h = take((size_t)sv::round16(R) * d.hidden * 4);
  w.n_cnt = sv::kCoopCounters;
  w.pcnt = take((size_t)w.n_cnt * 4);
  w.bar = w.pcnt;
  const size_t groups = (size_t)std::max(m->lm_groups, m->bf16 ? sv::kCUs : 0);
  w.lmp = take((size_t)R * groups * sizeof(sv::LmPartial));
  w.rstat = take((size_t)R * sizeof(sv::RowStat));
  w.dec = take((size_t)L * sizeof(sv::LaneDecision));
  w.racep = take((size_t)L * groups * 16);
  w.total = off;
  return w;
}

template <typename T>
T* at(void* base, size_t off) { return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off); }

bool valid_layer(const spec_layer_weights& w) {
  return w.norm1 && w.w_in && w.w_o && w.norm2 && w.w_gate && w.w_up && w.w_down;
}

int build_rowinfo(const spec_round* r, sv::RowInfo& ri) {
  if (!r || r->lanes < 1 || r->lanes > SPEC_MAX_LANES || !r->cols_host) return SPEC_E_INVAL;
  std::memset(&ri, 0, sizeof(ri));
  int R = 0;
  ri.L = r->lanes;
  for (int l = 0; l < r->lanes; ++l) {
    const int c = r->cols_host[l];
    if (c < 1 || c > SPEC_MAX_COLS) return SPEC_E_INVAL;
    if (R + c > SPEC_MAX_ROWS) return SPEC_E_INVAL;
    ri.lane_start[l] = (int16_t)R;
    ri.lane_cols[l] = (int8_t)c;
    for (int j = 0; j < c; ++j) {
      ri.row_lane[R + j] = (int8_t)l;
      ri.row_col[R + j] = (int8_t)j;
    }
    R += c;
  }
  ri.lane_start[r->lanes] = (int16_t)R;
  ri.R = R;
  return SPEC_OK;
}

int max_cols(const sv::RowInfo& ri) {
  int c = 0;
  for (int l = 0; l < ri.L; ++l) c = std::max(c, (int)ri.lane_cols[l]);
  return c;
}

// Common validation of a round; fills ri and the workspace layout.
// The window of the attention layer with this index among the attention layers: every
// window_global_every-th one keeps full attention (0 = none does).
int layer_window(const spec_model_desc& d, int attn_index) {
  const int g = d.window_global_every;
  if (d.sliding_window <= 0 || (g > 0 && attn_index % g == g - 1)) return 0;
  return d.sliding_window;
}

// The sampled bf16 head keeps a workgroup's vocabulary slice on chip: at most 64 tiles of
// 16 tokens per CU, and the head's bytes addressable by one buffer resource.
bool coop_head_fits(const spec_model* m) {
  const long long tiles = m->d.vocab / 16;
  return tiles <= 64LL * sv::kCUs && (long long)m->d.vocab * m->d.hidden * 2 <= 0x80000000LL;
}

// Greedy statistics of a bf16 head through the same one-workgroup-per-CU kernel (no grid
// barrier) when the head fits it on this device.
bool greedy_head_coop(const spec_model* m) {
  return m->bf16 && coop_head_fits(m) && (long long)m->d.vocab / 16 <= 64LL * sv::coop_grid();
}

// Validation of a round's arguments, the workspace aside; fills ri.
int validate_round(const spec_model* m, const spec_round* r, bool head_only, sv::RowInfo& ri) {
  if (!m) return SPEC_E_INVAL;
  int st = build_rowinfo(r, ri);
  if (st) return st;
  if (!r->tokens || !r->kv_len) return SPEC_E_INVAL;
  if (r->mode != SPEC_GREEDY && r->mode != SPEC_SAMPLED) return SPEC_E_INVAL;
  if (r->mode == SPEC_SAMPLED) {
    if (!r->q_probs || !(r->temperature > 0.f) || !std::isfinite(r->temperature)) return SPEC_E_INVAL;
  }
  if (r->mode == SPEC_SAMPLED && m->bf16 && !coop_head_fits(m)) return SPEC_E_UNSUPPORTED;
  if (r->counts && (!std::isfinite(r->presence_penalty) || !std::isfinite(r->frequency_penalty) ||
                    (reinterpret_cast<uintptr_t>(r->counts) & 15) != 0))
    return SPEC_E_INVAL;
  const int mb = head_only ? 1 : r->max_blocks;
  if (!head_only) {
    if (m->d.n_layers == 0) return SPEC_E_INVAL;
    if (m->n_attn) {
      if (!r->block_table || !r->k_pool || !r->v_pool || r->max_blocks < 1 || r->n_blocks < 1)
        return SPEC_E_INVAL;
      const int G = m->d.n_q_heads / m->d.n_kv_heads;
      const int mq = max_cols(ri) * G;
      if (mq > 64) return SPEC_E_UNSUPPORTED;   // a chunk partial holds 64 query rows
      if (!m->bf16 && (size_t)4 * mq * (m->d.head_dim + sv::kAttnPartPad) * 4 > 65536) return SPEC_E_UNSUPPORTED;
      if (r->kv_len_host) {
        for (int l = 0; l < r->lanes; ++l) {
          if (r->kv_len_host[l] < 0) return SPEC_E_INVAL;
          if ((long long)r->kv_len_host[l] + r->cols_host[l] > (long long)r->max_blocks * SPEC_KV_BLOCK)
            return SPEC_E_RANGE;
        }
      }
    }
    if (m->n_gdn && !r->gdn_state) return SPEC_E_UNSUPPORTED;
  }
  (void)mb;
  return SPEC_OK;
}

// Common validation of a round and of its workspace; fills ri and the workspace layout.
int check_round(const spec_model* m, const spec_round* r, bool head_only, sv::RowInfo& ri, WsLayout& w) {
  int st = validate_round(m, r, head_only, ri);
  if (st) return st;
  w = layout(m, ri.R, ri.L, head_only ? 1 : std::max(r->max_blocks, 1));
  if (!r->workspace) return SPEC_E_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(r->workspace) % kAlign) != 0) return SPEC_E_WORKSPACE;
  if (r->workspace_bytes < w.total) return SPEC_E_WORKSPACE;
  return SPEC_OK;
}

// ---------------------------------------------------------------- profiling
struct ProfScope {
  spec_model* m;
  hipStream_t st;
  bool on;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(const spec_model* mc, int cls, hipStream_t s) : m(const_cast<spec_model*>(mc)), st(s) {
    on = m->prof_class == cls && cls != SPEC_K_NONE && m->prof_seen++ % m->prof_every == 0;
    if (!on) return;
    while (m->prof_pool.size() < m->prof_used + 2) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) { on = false; return; }
      m->prof_pool.push_back(e);
    }
    a = m->prof_pool[m->prof_used++];
    b = m->prof_pool[m->prof_used++];
    hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (!on) return;
    hipEventRecord(b, st);
    m->prof_events.emplace_back(a, b);
  }
};

#define SV_CHECK(x)                 \
  do {                              \
    if ((x) != 0) return SPEC_E_HIP; \
  } while (0)

// ---------------------------------------------------------------- projections
// X: an fp32 model's float activations [R][K]; for a bf16 model the packed
// activation planes (hi, then lo when two_planes; one exact bf16 plane otherwise).
// W: packed fragments (bf16) or row-major [N][K] float.
// Q / cnt: the cut-unit pieces and counters of a balanced gate/up launch (null elsewhere).
int project(const spec_model* m, int cls, const void* X, bool two_planes, const void* W0, const void* W1, int R,
            int N, int K, int S, float* P, void* Y, hipStream_t st, float* Q = nullptr, int* cnt = nullptr) {
  ProfScope ps(m, cls, st);
  if (m->bf16) {
    sv::ProjParams p{};
    p.X = reinterpret_cast<const sv::bf16_t*>(X);
    p.xplane = sv::act_plane(R, K);
    p.W0 = reinterpret_cast<const sv::bf16_t*>(W0);
    p.W1 = reinterpret_cast<const sv::bf16_t*>(W1);
    p.R = R; p.N = N; p.K = K; p.S = S; p.tiles = (N + 15) / 16;
    p.P = P;
    p.Y = reinterpret_cast<sv::bf16_t*>(Y);
    p.yplane = sv::act_plane(R, N);
    p.Q = Q;
    p.cnt = cnt;
    return sv::launch_proj(p, W1 != nullptr, two_planes ? 2 : 1, st);
  }
  sv::GemmF32Params p{};
  p.X = reinterpret_cast<const float*>(X);
  p.W0 = reinterpret_cast<const float*>(W0);
  p.W1 = reinterpret_cast<const float*>(W1);
  p.R = R; p.N = N; p.K = K;
  p.P = P;
  p.Ya = reinterpret_cast<float*>(Y);
  return sv::launch_gemm_f32(p, W1 != nullptr, st);
}

// The decoder forward for all rows; leaves the final normed hidden states in ws.h.
int forward(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, hipStream_t st) {
  const spec_model_desc& d = m->d;
  void* ws = r->workspace;
  const bool bf = m->bf16;
  const int R = ri.R, H = d.hidden;
  float* x = at<float>(ws, w.x);
  void* h = at<void>(ws, w.h);
  float* P = at<float>(ws, w.P);
  const size_t ab = act_bytes(m);
  const bool rope = d.rope_theta != 0.f && m->n_attn > 0;
  if (rope) SV_CHECK(sv::launch_rope_table(r->kv_len, ri, d.head_dim, d.rope_theta, at<double>(ws, w.rope), st));
  const float* g0 = d.n_layers ? m->layers[0].w.norm1 : d.final_norm;
  SV_CHECK(sv::launch_embed_norm(r->tokens, d.embed, d.vocab, H, g0, d.rms_eps, x, h, ri, bf, at<int>(ws, w.pcnt),
                                 w.n_cnt, st));
  const size_t apool = (size_t)r->n_blocks * d.n_kv_heads * SPEC_KV_BLOCK * d.head_dim * ab;
  for (int i = 0; i < d.n_layers; ++i) {
    const Layer& L = m->layers[i];
    const float* gnext = i + 1 < d.n_layers ? m->layers[i + 1].w.norm1 : d.final_norm;
    int S_o;
    int Ko;
    if (L.kind == SPEC_LAYER_ATTN) {
      const int nq = d.n_q_heads, nkv = d.n_kv_heads, hd = d.head_dim;
      const int Nin = (nq + 2 * nkv) * hd;
      const int S_in = m->s_in_attn.S;
      SV_CHECK(project(m, SPEC_K_PROJ_IN, h, true, L.w.w_in, nullptr, R, Nin, H, S_in, P, nullptr, st));
      void* sk = at<char>(ws, w.stk) + (size_t)L.attn_index * w.stage_layer_elems * ab;
      void* svp = at<char>(ws, w.stv) + (size_t)L.attn_index * w.stage_layer_elems * ab;
      float* q = at<float>(ws, w.q);
      sv::AttnParams ap{};
      ap.q = q; ap.sk = sk; ap.sv = svp;
      ap.kpool = reinterpret_cast<const char*>(r->k_pool) + (size_t)L.attn_index * apool;
      ap.vpool = reinterpret_cast<const char*>(r->v_pool) + (size_t)L.attn_index * apool;
      if (bf) {
        // the attention kernel sums the QKV partials, rotates and stages the columns itself
        ap.P = P;
        ap.S = S_in;
        ap.rope = rope ? at<double>(ws, w.rope) : nullptr;
      } else {
        const sv::KvStage ks{r->kv_len, r->block_table, r->max_blocks, r->n_blocks, ap.kpool, ap.vpool};
        SV_CHECK(sv::launch_qkv_post(P, S_in, at<double>(ws, w.rope), rope ? 1 : 0, nq, nkv, hd, q, sk, svp, ks, ri,
                                     bf, st));
      }
      ap.block_table = r->block_table; ap.max_blocks = r->max_blocks; ap.n_blocks = r->n_blocks;
      ap.kv_len = r->kv_len;
      ap.nq = nq; ap.nkv = nkv; ap.G = nq / nkv; ap.d = hd;
      ap.chunk = m->chunk; ap.n_chunks = w.n_chunks;
      ap.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)hd));
      ap.part = at<float>(ws, w.apart);
      ap.ri = ri;
      ap.window = layer_window(m->d, L.attn_index);
      {
        ProfScope ps(m, SPEC_K_ATTN, st);
        SV_CHECK(sv::launch_attention(ap, bf, st));
      }
      SV_CHECK(sv::launch_attn_combine(ap, at<void>(ws, w.o), bf, st));
      S_o = m->s_o_attn.S;
      Ko = nq * hd;
    } else {
      const int hg = d.gdn_heads, dg = d.gdn_dim;
      const int Nin = 3 * hg * dg + 2 * hg;
      const int S_in = m->s_in_gdn.S;
      SV_CHECK(project(m, SPEC_K_PROJ_IN, h, true, L.w.w_in, nullptr, R, Nin, H, S_in, P, nullptr, st));
      float* stage = at<float>(ws, w.gst) + (size_t)L.gdn_index * w.gst_layer_floats;
      {
        ProfScope ps(m, SPEC_K_GDN, st);
        SV_CHECK(sv::launch_gdn_verify(P, S_in, hg, dg, r->gdn_state, m->n_gdn, L.gdn_index, stage,
                                       at<void>(ws, w.o), ri, bf, st));
      }
      S_o = m->s_o_gdn.S;
      Ko = hg * dg;
    }
    SV_CHECK(project(m, SPEC_K_PROJ_O, at<void>(ws, w.o), true, L.w.w_o, nullptr, R, H, Ko, S_o, P, nullptr, st));
    SV_CHECK(sv::launch_resid_norm(P, S_o, x, H, L.w.norm2, d.rms_eps, h, ri, bf, st));
    SV_CHECK(project(m, SPEC_K_GATE_UP, h, true, L.w.w_gate, L.w.w_up, R, d.ffn, H, 1, nullptr, at<void>(ws, w.a),
                     st, at<float>(ws, w.pieces), at<int>(ws, w.pcnt)));
    SV_CHECK(project(m, SPEC_K_DOWN, at<void>(ws, w.a), true, L.w.w_down, nullptr, R, H, d.ffn, m->s_down.S, P,
                     nullptr, st));
    SV_CHECK(sv::launch_resid_norm(P, m->s_down.S, x, H, gnext, d.rms_eps, h, ri, bf, st));
  }
  return SPEC_OK;
}

int lm_stats(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, hipStream_t st) {
  sv::LmParams p{};
  p.X = at<void>(r->workspace, w.h);
  p.xplane = sv::act_plane(ri.R, m->d.hidden);
  p.xs = m->d.n_layers == 0 ? 1 : 2;
  p.W = m->d.lm_head;
  p.R = ri.R; p.V = m->d.vocab; p.H = m->d.hidden;
  p.groups = m->lm_groups;
  p.tokens = r->tokens;
  p.kv_len = r->kv_len;
  p.sampled = r->mode == SPEC_SAMPLED;
  p.inv_t = p.sampled ? 1.0f / r->temperature : 1.0f;
  p.key0 = (uint32_t)(r->seed & 0xffffffffu);
  p.key1 = (uint32_t)(r->seed >> 32);
  p.part = at<sv::LmPartial>(r->workspace, w.lmp);
  p.ri = ri;
  p.counts = r->counts;
  p.presence = r->presence_penalty;
  p.frequency = r->frequency_penalty;
  p.bar = at<int>(r->workspace, w.bar);
  p.spin_limit = m->barrier_spin;
  p.rstat = at<sv::RowStat>(r->workspace, w.rstat);
  p.dec = at<sv::LaneDecision>(r->workspace, w.dec);
  p.racep = at<float>(r->workspace, w.racep);
  p.q = r->q_probs;
  ProfScope ps(m, SPEC_K_LM_HEAD, st);
  if (m->bf16 && (p.sampled || greedy_head_coop(m))) {
    // one workgroup per CU over a vocabulary slice each: sampled, statistics, decisions and
    // residual race in one cooperative launch; greedy, the per-workgroup statistics only
    const int rc = sv::launch_lmhead_coop(p, sv::coop_grid(), st);
    return rc == 0 ? SPEC_OK : (rc == -2 ? SPEC_E_UNSUPPORTED : SPEC_E_HIP);
  }
  return sv::launch_lmhead(p, m->bf16, st) ? SPEC_E_HIP : SPEC_OK;
}

int run_head(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, const void* hidden,
             hipStream_t s);
int run_accept(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, int32_t* committed,
               int32_t* out_tokens, spec_row_stat* row_stats, hipStream_t s);

}  // namespace

extern "C" {

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "ok";
    case SPEC_E_INVAL: return "invalid argument";
    case SPEC_E_RANGE: return "round exceeds the lane's block table";
    case SPEC_E_UNSUPPORTED: return "unsupported shape or configuration";
    case SPEC_E_WORKSPACE: return "workspace missing, misaligned or too small";
    case SPEC_E_HIP: return "HIP runtime error";
    case SPEC_E_SCRATCH: return "round needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int spec_plan_drafts(int k, int row_budget, int lanes) {
  if (lanes <= 0 || k < 0 || row_budget < 0) return SPEC_E_INVAL;
  const int rows = row_budget == 0 ? 8 : row_budget;
  return std::max(0, std::min(k, rows / lanes - 1));
}

int spec_window_live_block(int kv_len, int window) {
  if (kv_len < 0 || window < 0) return SPEC_E_INVAL;
  if (window == 0) return 0;
  // windowed layers read from the 64-position stage that holds the lowest window start
  return std::max(0, kv_len - window + 1) / 64 * (64 / SPEC_KV_BLOCK);
}

int spec_model_create(const spec_model_desc* desc, spec_model** out) {
  if (!desc || !out) return SPEC_E_INVAL;
  *out = nullptr;
  const spec_model_desc& d = *desc;
  if (d.n_layers < 0 || d.hidden <= 0 || d.vocab <= 0 || (d.vocab % 16) != 0) return SPEC_E_INVAL;
  if (d.dtype != SPEC_F32 && d.dtype != SPEC_BF16) return SPEC_E_INVAL;
  if (d.kv_block != SPEC_KV_BLOCK) return SPEC_E_UNSUPPORTED;
  if (!d.lm_head) return SPEC_E_INVAL;
  if (!(d.rms_eps >= 0.f) || !(d.rope_theta >= 0.f)) return SPEC_E_INVAL;
  if (d.sliding_window < 0 || d.window_global_every < 0) return SPEC_E_INVAL;
  const bool bf = d.dtype == SPEC_BF16;
  if (bf && (d.hidden % 256) != 0) return SPEC_E_UNSUPPORTED;
  if ((d.hidden % 4) != 0 || d.hidden > 8192) return SPEC_E_UNSUPPORTED;
  const int chunk = d.attn_chunk == 0 ? kDefaultChunk : d.attn_chunk;
  if (chunk < 256 || (chunk % 256) != 0 || chunk > sv::kMaxChunk) return SPEC_E_UNSUPPORTED;
  spec_model* m = new (std::nothrow) spec_model();
  if (!m) return SPEC_E_INVAL;
  m->d = d;
  m->bf16 = bf;
  m->chunk = chunk;
  if (d.n_layers > 0) {
    if (!d.layer_kind || !d.layers || !d.embed || !d.final_norm || d.ffn <= 0) { delete m; return SPEC_E_INVAL; }
    if (bf && (d.ffn % 256) != 0) { delete m; return SPEC_E_UNSUPPORTED; }
    m->kinds.assign(d.layer_kind, d.layer_kind + d.n_layers);
    for (int i = 0; i < d.n_layers; ++i) {
      Layer L{};
      L.kind = d.layer_kind[i];
      L.w = d.layers[i];
      L.attn_index = L.gdn_index = -1;
      if (!valid_layer(L.w)) { delete m; return SPEC_E_INVAL; }
      if (L.kind == SPEC_LAYER_ATTN) L.attn_index = m->n_attn++;
      else if (L.kind == SPEC_LAYER_GDN) L.gdn_index = m->n_gdn++;
      else { delete m; return SPEC_E_INVAL; }
      m->layers.push_back(L);
    }
    if (m->n_attn) {
      if (d.n_q_heads <= 0 || d.n_kv_heads <= 0 || (d.n_q_heads % d.n_kv_heads) != 0) { delete m; return SPEC_E_INVAL; }
      if (d.head_dim <= 0 || (d.head_dim % 2) != 0) { delete m; return SPEC_E_INVAL; }
      if (bf && (d.head_dim != 128 || ((d.n_q_heads * d.head_dim) % 256) != 0)) { delete m; return SPEC_E_UNSUPPORTED; }
      if (!bf && (d.head_dim > 128 || (d.head_dim % 8) != 0)) { delete m; return SPEC_E_UNSUPPORTED; }
    }
    if (m->n_gdn) {
      if (d.gdn_heads <= 0 || d.gdn_dim != 128) { delete m; return SPEC_E_UNSUPPORTED; }
      if (bf && ((d.gdn_heads * d.gdn_dim) % 256) != 0) { delete m; return SPEC_E_UNSUPPORTED; }
    }
  }
  m->d.layer_kind = m->kinds.empty() ? nullptr : m->kinds.data();
  m->d.layers = nullptr;   // per-layer weights live in m->layers
  const int H = d.hidden;
  if (m->n_attn) {
    m->s_in_attn.S = split_for(m, (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim, H, false, 4);
    m->s_o_attn.S = split_for(m, H, d.n_q_heads * d.head_dim, false);
  }
  if (m->n_gdn) {
    m->s_in_gdn.S = split_for(m, 3 * d.gdn_heads * d.gdn_dim + 2 * d.gdn_heads, H, false, 4);
    m->s_o_gdn.S = split_for(m, H, d.gdn_heads * d.gdn_dim, false);
  }
  if (d.n_layers) {
    m->s_gateup.S = 1;
    m->s_down.S = split_for(m, H, d.ffn, false);
  }
  m->lm_groups = sv::lmhead_groups(d.vocab, bf);
  *out = m;
  return SPEC_OK;
}

void spec_model_destroy(spec_model* m) {
  if (!m) return;
  for (hipEvent_t e : m->prof_pool) hipEventDestroy(e);
  delete m;
}

int64_t spec_workspace_bytes(const spec_model* m, int max_lanes, int max_cols, int max_blocks) {
  if (!m || max_lanes < 1 || max_lanes > SPEC_MAX_LANES || max_cols < 1 || max_cols > SPEC_MAX_COLS ||
      max_blocks < 0)
    return SPEC_E_INVAL;
  const int R = std::min(SPEC_MAX_ROWS, max_lanes * max_cols);
  return (int64_t)layout(m, R, max_lanes, std::max(max_blocks, 1)).total;
}

int spec_verify_round(const spec_model* m, const spec_round* r, void* stream) {
  sv::RowInfo ri;
  WsLayout w;
  int st = check_round(m, r, false, ri, w);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = forward(m, r, ri, w, s);
  if (st) return st;
  return lm_stats(m, r, ri, w, s);
}

int spec_verify_head(const spec_model* m, const spec_round* r, const void* hidden, void* stream) {
  sv::RowInfo ri;
  WsLayout w;
  if (!hidden) return SPEC_E_INVAL;
  int st = check_round(m, r, true, ri, w);
  if (st) return st;
  return run_head(m, r, ri, w, hidden, reinterpret_cast<hipStream_t>(stream));
}

int spec_accept(const spec_model* m, const spec_round* r, int32_t* committed, int32_t* out_tokens,
                spec_row_stat* row_stats, void* stream) {
  sv::RowInfo ri;
  WsLayout w;
  if (!committed || !out_tokens) return SPEC_E_INVAL;
  const bool head_only = !m || m->d.n_layers == 0;
  int st = check_round(m, r, head_only, ri, w);
  if (st) return st;
  return run_accept(m, r, ri, w, committed, out_tokens, row_stats, reinterpret_cast<hipStream_t>(stream));
}

int spec_verify_head_noalloc(const spec_model* m, const spec_round* r, const void* hidden, int32_t* committed,
                             int32_t* out_tokens, spec_row_stat* row_stats, void* stream) {
  sv::RowInfo ri;
  if (!hidden || !committed || !out_tokens) return SPEC_E_INVAL;
  int st = validate_round(m, r, true, ri);
  if (st) return st;
  const WsLayout w = head_layout(m, ri.R, ri.L);
  if (w.total > sv::kStaticScratchBytes) return SPEC_E_SCRATCH;
  void* scr = nullptr;
  size_t scr_bytes = 0;
  if (sv::static_scratch(&scr, &scr_bytes) || scr_bytes < w.total) return SPEC_E_HIP;
  spec_round rs = *r;   // the same round on the library's scratch
  rs.workspace = scr;
  rs.workspace_bytes = scr_bytes;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = run_head(m, &rs, ri, w, hidden, s);
  if (st) return st;
  return run_accept(m, &rs, ri, w, committed, out_tokens, row_stats, s);
}

}  // extern "C"

namespace {

// The LM head and row statistics on caller-given hidden states (spec_verify_head), on the
// workspace of r laid out by w.
int run_head(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, const void* hidden,
             hipStream_t s) {
  if (m->bf16)
    SV_CHECK(sv::launch_pack_rows(hidden, at<void>(r->workspace, w.h), ri.R, m->d.hidden,
                                  sv::act_plane(ri.R, m->d.hidden), m->d.n_layers == 0 ? 1 : 2,
                                  at<int>(r->workspace, w.pcnt), w.n_cnt, s));
  else
    SV_CHECK(sv::launch_copy_rows(hidden, at<void>(r->workspace, w.h), (size_t)ri.R * m->d.hidden * 4, s));
  return lm_stats(m, r, ri, w, s);
}

// Acceptance (spec_accept) on the workspace of r laid out by w.
int run_accept(const spec_model* m, const spec_round* r, const sv::RowInfo& ri, const WsLayout& w, int32_t* committed,
               int32_t* out_tokens, spec_row_stat* row_stats, hipStream_t s) {
  void* ws = r->workspace;
  const bool sampled = r->mode == SPEC_SAMPLED;
  const float inv_t = sampled ? 1.0f / r->temperature : 1.0f;
  const uint32_t k0 = (uint32_t)(r->seed & 0xffffffffu), k1 = (uint32_t)(r->seed >> 32);
  if (sampled && m->bf16) {   // the head's cooperative launch has taken the decisions and run the races
    SV_CHECK(sv::launch_accept_coop(at<sv::RowStat>(ws, w.rstat), at<sv::LaneDecision>(ws, w.dec),
                                    at<float>(ws, w.racep), at<int>(ws, w.bar), r->tokens, inv_t, committed,
                                    out_tokens, row_stats, ri, s));
    return SPEC_OK;
  }
  const int groups = greedy_head_coop(m) ? sv::coop_grid() : m->lm_groups;   // the head's partials per row
  SV_CHECK(sv::launch_row_reduce(at<sv::LmPartial>(ws, w.lmp), groups, ri.R, inv_t, at<sv::RowStat>(ws, w.rstat),
                                 row_stats, s));
  SV_CHECK(sv::launch_lane_accept(at<sv::RowStat>(ws, w.rstat), r->tokens, r->kv_len, r->q_probs, m->d.vocab,
                                  sampled ? 1 : 0, inv_t, k0, k1, at<sv::LaneDecision>(ws, w.dec), committed,
                                  out_tokens, ri, s));
  if (sampled) {
    sv::RaceParams p{};   // fp32 model: the race recomputes the rejected row's logits
    p.X = at<void>(ws, w.h);
    p.W = m->d.lm_head;
    p.R = ri.R; p.V = m->d.vocab; p.H = m->d.hidden; p.L = ri.L;
    p.groups = m->lm_groups;
    p.q = r->q_probs;
    p.kv_len = r->kv_len;
    p.inv_t = inv_t;
    p.key0 = k0; p.key1 = k1;
    p.dec = at<sv::LaneDecision>(ws, w.dec);
    p.part = at<float>(ws, w.racep);
    p.ri = ri;
    p.tokens = r->tokens;
    p.counts = r->counts;
    p.presence = r->presence_penalty;
    p.frequency = r->frequency_penalty;
    SV_CHECK(sv::launch_race(p, s));
    SV_CHECK(sv::launch_race_finish(at<float>(ws, w.racep), m->lm_groups, at<sv::LaneDecision>(ws, w.dec),
                                    out_tokens, ri, s));
  }
  return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_commit(const spec_model* m, const spec_round* r, const int32_t* committed, void* stream) {
  sv::RowInfo ri;
  WsLayout w;
  if (!committed) return SPEC_E_INVAL;
  int st = check_round(m, r, false, ri, w);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const spec_model_desc& d = m->d;
  if (m->n_attn)
    SV_CHECK(sv::launch_commit_kv(committed, r->kv_len, r->block_table, r->max_blocks, r->n_blocks, r->k_pool,
                                  r->v_pool, m->n_attn, d.n_kv_heads, d.head_dim, at<void>(r->workspace, w.stk),
                                  at<void>(r->workspace, w.stv), w.stage_layer_elems, ri, m->bf16, s));
  if (m->n_gdn)
    SV_CHECK(sv::launch_gdn_replay(committed, r->gdn_state, m->n_gdn, d.gdn_heads, d.gdn_dim,
                                   at<float>(r->workspace, w.gst), w.gst_layer_floats, ri, s));
  SV_CHECK(sv::launch_kvlen_update(committed, r->kv_len, ri, s));
  return SPEC_OK;
}

int spec_debug_logits(const spec_model* m, const spec_round* r, float* logits, void* stream) {
  sv::RowInfo ri;
  WsLayout w;
  if (!logits) return SPEC_E_INVAL;
  int st = check_round(m, r, false, ri, w);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  st = forward(m, r, ri, w, s);
  if (st) return st;
  // one split: the same accumulation chain as the LM-head kernel
  return project(m, SPEC_K_NONE, at<void>(r->workspace, w.h), true, m->d.lm_head, nullptr, ri.R, m->d.vocab,
                 m->d.hidden, 1, logits, nullptr, s)
             ? SPEC_E_HIP
             : SPEC_OK;
}

int spec_debug_gemm(const spec_model* m, const void* X, const void* W, float* Y, int R, int N, int K,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (!m || !X || !W || !Y || R < 1 || R > SPEC_MAX_ROWS || N < 1 || K < 1) return SPEC_E_INVAL;
  if (m->bf16 && (K % 256) != 0) return SPEC_E_UNSUPPORTED;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int S = split_for(m, N, K, false);
  if (!m->bf16) return project(m, SPEC_K_PROJ_IN, X, false, W, nullptr, R, N, K, 1, Y, nullptr, s) ? SPEC_E_HIP : SPEC_OK;
  // bf16: the rows are packed into the workspace, then partials follow
  const size_t xbytes = align_up(sv::act_plane(R, K) * 2);
  const size_t need = xbytes + (S > 1 ? (size_t)S * R * N * 4 : 0);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) % kAlign) != 0)
    return SPEC_E_WORKSPACE;
  void* xp = workspace;
  SV_CHECK(sv::launch_pack_rows(X, xp, R, K, sv::act_plane(R, K), 1, nullptr, 0, s));
  if (S == 1) return project(m, SPEC_K_PROJ_IN, xp, false, W, nullptr, R, N, K, 1, Y, nullptr, s) ? SPEC_E_HIP : SPEC_OK;
  float* P = at<float>(workspace, xbytes);
  SV_CHECK(project(m, SPEC_K_PROJ_IN, xp, false, W, nullptr, R, N, K, S, P, nullptr, s));
  SV_CHECK(sv::launch_sum_partials(P, S, (size_t)R * N, Y, s));
  return SPEC_OK;
}

int64_t spec_packed_weight_bytes(int N, int K) {
  if (N < 1 || K < 256 || (K % 256) != 0) return SPEC_E_INVAL;
  return (int64_t)sv::round16(N) * K * 2;
}

int spec_pack_weight(const void* src, void* dst, int N, int K, void* stream) {
  if (!src || !dst || N < 1 || K < 256 || (K % 256) != 0) return SPEC_E_INVAL;
  if (src == dst) return SPEC_E_INVAL;
  return sv::launch_pack_weight(src, dst, N, K, reinterpret_cast<hipStream_t>(stream)) ? SPEC_E_HIP : SPEC_OK;
}

// ---------------------------------------------------------------- miss back-off (host)
constexpr int kMissPasses = 4, kFirstWait = 16, kMaxWait = 256;

int spec_backoff_init(spec_backoff* st, int n) {
  if (!st || n < 1 || n > SPEC_MAX_LANES) return SPEC_E_INVAL;
  for (int i = 0; i < n; ++i) st[i] = spec_backoff{0, kFirstWait, 0, 1};
  return SPEC_OK;
}

int spec_backoff_call(spec_backoff* st, int n, int k, int row_budget, int32_t* drafts) {
  if (!st || !drafts || n < 1 || n > SPEC_MAX_LANES) return SPEC_E_INVAL;
  const int plan = spec_plan_drafts(k, row_budget, n);
  if (plan < 0) return plan;
  bool any = false;
  for (int i = 0; i < n; ++i) {
    st[i].may_guess = st[i].wait_left == 0;
    any = any || st[i].may_guess;
  }
  const bool speculates = any && plan > 0;
  for (int i = 0; i < n; ++i) drafts[i] = speculates && st[i].may_guess ? plan : 0;
  return speculates ? 1 : 0;
}

int spec_backoff_pass(spec_backoff* st, int n, const int32_t* kept, int speculates) {
  if (!st || !kept || n < 1 || n > SPEC_MAX_LANES) return SPEC_E_INVAL;
  for (int i = 0; i < n; ++i) {
    spec_backoff& s = st[i];
    if (speculates && s.may_guess && s.wait_left == 0) {
      if (kept[i] > 0) {          // a kept guess: the count clears, the next wait is 16 again
        s.miss_run = 0;
        s.wait_len = kFirstWait;
      } else if (++s.miss_run == kMissPasses) {
        s.miss_run = 0;
        s.wait_left = s.wait_len;
        s.wait_len = std::min(2 * s.wait_len, kMaxWait);
      }
    } else if (s.wait_left > 0) {  // waiting: the pass counts toward the wait, kept or not
      --s.wait_left;
    }
  }
  return SPEC_OK;
}

static_assert(SPEC_MAX_NGRAM == sv::kMaxNgram, "n-gram bound of the header and the kernels");

int spec_ngram_draft(const int32_t* history, const int32_t* hist_len, int lanes, int max_len, int k, int n_max,
                     int n_min, int32_t* tokens, int32_t* n_match, void* stream) {
  if (!history || !hist_len || !tokens || !n_match) return SPEC_E_INVAL;
  if (lanes < 1 || lanes > SPEC_MAX_LANES || max_len < 1 || k < 0 || k >= SPEC_MAX_COLS) return SPEC_E_INVAL;
  if (n_min < 1 || n_max < n_min || n_max > SPEC_MAX_NGRAM) return SPEC_E_INVAL;
  return sv::launch_ngram_draft(history, hist_len, lanes, max_len, k, n_max, n_min, tokens, n_match,
                                reinterpret_cast<hipStream_t>(stream))
             ? SPEC_E_HIP
             : SPEC_OK;
}

int spec_counts_add(int32_t* counts, int vocab, int lanes, const int32_t* committed, const int32_t* out_tokens,
                    int out_stride, void* stream) {
  if (!counts || !committed || !out_tokens) return SPEC_E_INVAL;
  if (lanes < 1 || lanes > SPEC_MAX_LANES || vocab < 1 || out_stride < 1) return SPEC_E_INVAL;
  return sv::launch_counts_add(counts, vocab, lanes, committed, out_tokens, out_stride,
                               reinterpret_cast<hipStream_t>(stream))
             ? SPEC_E_HIP
             : SPEC_OK;
}

int spec_history_append(int32_t* history, int32_t* hist_len, int lanes, int max_len, const int32_t* committed,
                        const int32_t* out_tokens, int out_stride, void* stream) {
  if (!history || !hist_len || !committed || !out_tokens) return SPEC_E_INVAL;
  if (lanes < 1 || lanes > SPEC_MAX_LANES || max_len < 1 || out_stride < 1) return SPEC_E_INVAL;
  return sv::launch_history_append(history, hist_len, lanes, max_len, committed, out_tokens, out_stride,
                                   reinterpret_cast<hipStream_t>(stream))
             ? SPEC_E_HIP
             : SPEC_OK;
}

int spec_profile_enable(spec_model* m, int kernel_class, int every) {
  if (!m || kernel_class < SPEC_K_NONE || kernel_class >= SPEC_K_COUNT || every < 1) return SPEC_E_INVAL;
  m->prof_class = kernel_class;
  m->prof_every = every;
  m->prof_seen = 0;
  m->prof_events.clear();
  m->prof_used = 0;
  return SPEC_OK;
}

int spec_debug_barrier_spin(spec_model* m, int polls) {
  if (!m || polls < 0) return SPEC_E_INVAL;
  m->barrier_spin = polls;
  return SPEC_OK;
}

int spec_profile_collect(spec_model* m, double* total_ms, int* launches) {
  if (!m || !total_ms || !launches) return SPEC_E_INVAL;
  double t = 0.0;
  for (auto& ev : m->prof_events) {
    if (hipEventSynchronize(ev.second) != hipSuccess) return SPEC_E_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess) return SPEC_E_HIP;
    t += ms;
  }
  *total_ms = t;
  *launches = (int)m->prof_events.size();
  return SPEC_OK;
}

}  // extern "C"
