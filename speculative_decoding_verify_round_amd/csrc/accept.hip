// Acceptance kernels of the verify round (gfx950).
//
// Greedy ("Speculative decoding", gpillon.github.io/ignis, "One round, step by
// step", step 4; "Draft heads and speculative decoding",
// research.strata2signal.com, "Guess, then check"): keep drafts while each
// equals the model's own argmax at the row before it; the model's token at the
// first mismatch, or after the last draft, ends the committed run (1 .. k+1).
//
// Sampled (the textbook rule that page cites, Leviathan et al. Def. 3.7):
// draft d_i is kept iff u * q_i(d_i) < p_{i-1}(d_i), u the Philox uniform at
// (seed; position kv_len + i, lane, accept); the first rejection draws from
// max(0, p_{i-1} - q_i) by the exponential race (k_race_*), and a fully kept
// lane takes its bonus token from p_k (race winner of its last row, computed
// with the LM head).
#include "common.hpp"
#include "launch.hpp"

namespace sv {

// Reduce the LM-head partials of one row in group order (a fixed tree of 256 -> 1).
__global__ __launch_bounds__(256) void k_row_reduce(const LmPartial* part, int groups, float inv_t, RowStat* rs,
                                                     spec_row_stat_dev* user) {
  __shared__ float sm[256], sse[256], szn[256], sgk[256];
  __shared__ int sarg[256], sgi[256];
  const int r = blockIdx.x, t = threadIdx.x;
  const int g0 = (int)((long long)t * groups / 256), g1 = (int)((long long)(t + 1) * groups / 256);
  float m = -INFINITY, se = 0.f, zn = NAN, gk = -INFINITY;
  int arg = 0x7fffffff, gi = 0x7fffffff;
  auto merge = [&](float bm, float bse, int barg, float bzn, float bgk, int bgi) {
    float om = m; int oa = arg;
    if (better(bm, barg, m, arg)) { om = bm; oa = barg; }
    const float fa = m == -INFINITY ? 0.f : expf((m - om) * inv_t);
    const float fb = bm == -INFINITY ? 0.f : expf((bm - om) * inv_t);
    se = se * fa + bse * fb;
    m = om; arg = oa;
    if (isnan(zn)) zn = bzn;
    if (better(bgk, bgi, gk, gi)) { gk = bgk; gi = bgi; }
  };
  for (int g = g0; g < g1; ++g) {
    const LmPartial pp = part[(size_t)r * groups + g];
    merge(pp.m, pp.se, pp.arg, pp.zn, pp.gk, pp.gi);
  }
  sm[t] = m; sse[t] = se; sarg[t] = arg; szn[t] = zn; sgk[t] = gk; sgi[t] = gi;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      m = sm[t]; se = sse[t]; arg = sarg[t]; zn = szn[t]; gk = sgk[t]; gi = sgi[t];
      merge(sm[t + w], sse[t + w], sarg[t + w], szn[t + w], sgk[t + w], sgi[t + w]);
      sm[t] = m; sse[t] = se; sarg[t] = arg; szn[t] = zn; sgk[t] = gk; sgi[t] = gi;
    }
    __syncthreads();
  }
  if (t == 0) {
    RowStat o;
    o.m = sm[0]; o.se = sse[0]; o.arg = sarg[0]; o.zn = szn[0]; o.gk = sgk[0]; o.gi = sgi[0];
    o.pad0 = o.pad1 = 0;
    rs[r] = o;
    if (user) {
      user[r].max_logit = o.m;
      user[r].lse = o.m * inv_t + logf(o.se);
      user[r].argmax = o.arg;
      user[r].z_next = o.zn;
    }
  }
}

int launch_row_reduce(const LmPartial* part, int groups, int R, float inv_t, RowStat* rs, void* user_stats,
                      hipStream_t st) {
  hipLaunchKernelGGL(k_row_reduce, dim3(R), dim3(256), 0, st, part, groups, inv_t, rs,
                     reinterpret_cast<spec_row_stat_dev*>(user_stats));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// One thread per lane walks its drafts.
__global__ void k_lane_accept(const RowStat* rs, const int32_t* tokens, const int32_t* kv_len, const float* q, int V,
                              int sampled, float inv_t, uint32_t key0, uint32_t key1, LaneDecision* dec,
                              int32_t* committed, int32_t* out, RowInfo ri) {
  const int l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= ri.L) return;
  const int r0 = ri.lane_start[l], k = ri.lane_cols[l] - 1;
  int32_t* o = out + (size_t)l * kMaxCols;
  LaneDecision d;
  d.resid_row = -1; d.resid_col = 0; d.pad = 0; d.m = 0.f; d.se = 1.f; d.pad2 = d.pad3 = 0.f;
  if (!sampled) {
    int a = 0;
    while (a < k && tokens[r0 + a + 1] == rs[r0 + a].arg) {
      o[a] = tokens[r0 + a + 1];
      ++a;
    }
    o[a] = rs[r0 + a].arg;
    d.committed = a + 1;
  } else {
    auto qd = [&](int r) {
      const int t = tokens[r];
      return (t >= 0 && t < V) ? q[(size_t)r * V + t] : 0.f;
    };
    d = decide_sampled(rs, tokens, kv_len, qd, inv_t, key0, key1, ri, l, o);
  }
  dec[l] = d;
  committed[l] = d.committed;
}

int launch_lane_accept(const RowStat* rs, const int32_t* tokens, const int32_t* kv_len, const float* q, int V,
                       int sampled, float inv_t, uint32_t key0, uint32_t key1, LaneDecision* dec,
                       int32_t* committed, int32_t* out, const RowInfo& ri, hipStream_t st) {
  hipLaunchKernelGGL(k_lane_accept, dim3(1), dim3(64), 0, st, rs, tokens, kv_len, q, V, sampled, inv_t, key0, key1,
                     dec, committed, out, ri);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Reduce the race partials of each rejecting lane in group order (min key, lowest index).
__global__ __launch_bounds__(256) void k_race_finish(const float* part, int groups, const LaneDecision* dec,
                                                      int32_t* out) {
  __shared__ float sk[256], sf[256];
  __shared__ int si[256], sfi[256];
  const int l = blockIdx.x, t = threadIdx.x;
  const LaneDecision d = dec[l];
  if (d.resid_row < 0) return;
  float k = INFINITY, f = INFINITY;
  int ki = 0x7fffffff, fi = 0x7fffffff;
  for (int g = t; g < groups; g += 256) {
    const float* pp = part + ((size_t)l * groups + g) * 4;
    const float bk = pp[0], bf = pp[2];
    const int bi = __float_as_int(pp[1]), bfi = __float_as_int(pp[3]);
    if (bk < k || (bk == k && bi < ki)) { k = bk; ki = bi; }
    if (bf < f || (bf == f && bfi < fi)) { f = bf; fi = bfi; }
  }
  sk[t] = k; si[t] = ki; sf[t] = f; sfi[t] = fi;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      if (sk[t + w] < sk[t] || (sk[t + w] == sk[t] && si[t + w] < si[t])) { sk[t] = sk[t + w]; si[t] = si[t + w]; }
      if (sf[t + w] < sf[t] || (sf[t + w] == sf[t] && sfi[t + w] < sfi[t])) { sf[t] = sf[t + w]; sfi[t] = sfi[t + w]; }
    }
    __syncthreads();
  }
  if (t == 0) {
    const int x = sk[0] < INFINITY ? si[0] : sfi[0];   // residual vanished: draw from p
    out[(size_t)l * kMaxCols + d.resid_col - 1] = x;
  }
}

int launch_race_finish(const float* part, int groups, const LaneDecision* dec, int32_t* out,
                       const RowInfo& ri, hipStream_t st) {
  hipLaunchKernelGGL(k_race_finish, dim3(ri.L), dim3(256), 0, st, part, groups, dec, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Sampled rounds of a bf16 model: the LM head's cooperative launch has already reduced
// the row statistics, taken every lane's decision and run its draw (residual or bonus
// race) over each workgroup's vocabulary slice (k_lmhead_coop).  Per lane: the user row
// statistics, the race partials reduced in workgroup order (min key, lowest index), the
// committed run.
// bar[2] set means a grid barrier of the head ran out of time: committed = 0 flags the
// round as failed.
__global__ __launch_bounds__(256) void k_accept_coop(const RowStat* rs, const LaneDecision* dec, const float* part,
                                                      const int* bar, const int32_t* tokens, float inv_t,
                                                      int32_t* committed, int32_t* out, spec_row_stat_dev* user,
                                                      RowInfo ri) {
  __shared__ float sk[256], sf[256];
  __shared__ int si[256], sfi[256];
  const int l = blockIdx.x, t = threadIdx.x;
  const int r0 = ri.lane_start[l], k = ri.lane_cols[l] - 1;
  const LaneDecision d = dec[l];
  const int groups = min(max(bar[3], 0), kCUs);
  if (user && t <= k) {
    const RowStat s = rs[r0 + t];
    user[r0 + t].max_logit = s.m;
    user[r0 + t].lse = s.m * inv_t + logf(s.se);
    user[r0 + t].argmax = s.arg;
    user[r0 + t].z_next = s.zn;
  }
  int x;
  {   // the lane's draw: the residual race, or the bonus race when every draft was kept
    float kk = INFINITY, f = INFINITY;
    int ki = 0x7fffffff, fi = 0x7fffffff;
    for (int g = t; g < groups; g += 256) {
      const float* pp = part + ((size_t)l * groups + g) * 4;
      const float bk = pp[0], bf = pp[2];
      const int bi = __float_as_int(pp[1]), bfi = __float_as_int(pp[3]);
      if (bk < kk || (bk == kk && bi < ki)) { kk = bk; ki = bi; }
      if (bf < f || (bf == f && bfi < fi)) { f = bf; fi = bfi; }
    }
    sk[t] = kk; si[t] = ki; sf[t] = f; sfi[t] = fi;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
      if (t < w) {
        if (sk[t + w] < sk[t] || (sk[t + w] == sk[t] && si[t + w] < si[t])) { sk[t] = sk[t + w]; si[t] = si[t + w]; }
        if (sf[t + w] < sf[t] || (sf[t + w] == sf[t] && sfi[t + w] < sfi[t])) { sf[t] = sf[t + w]; sfi[t] = sfi[t + w]; }
      }
      __syncthreads();
    }
    x = sk[0] < INFINITY ? si[0] : sfi[0];   // residual vanished: draw from p
  }
  if (t == 0) {
    const bool failed = bar[2] != 0;
    const int c = failed ? 0 : d.committed;
    committed[l] = c;
    if (!failed) {
      int32_t* o = out + (size_t)l * kMaxCols;
      for (int i = 0; i + 1 < c; ++i) o[i] = tokens[r0 + i + 1];
      o[c - 1] = x;
    }
  }
}

int launch_accept_coop(const RowStat* rs, const LaneDecision* dec, const float* part, const int* bar,
                       const int32_t* tokens, float inv_t, int32_t* committed, int32_t* out, void* user_stats,
                       const RowInfo& ri, hipStream_t st) {
  hipLaunchKernelGGL(k_accept_coop, dim3(ri.L), dim3(256), 0, st, rs, dec, part, bar, tokens, inv_t, committed, out,
                     reinterpret_cast<spec_row_stat_dev*>(user_stats), ri);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace sv
