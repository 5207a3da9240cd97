// Attention kernels: parameter block and host launchers.
#pragma once

#include "common.hpp"

namespace ispa {

// One segment of a key group as the kernels see it.
struct AttnSeg {
  const void* k;
  const void* v;
  int64_t n;
  int64_t ks;  // row strides in elements
  int64_t vs;
};

// One unit of key work: keys [kbeg, kend) of group `group` (positions in the
// concatenation of that group's segments), written as normalised o and lse.
struct AttnJob {
  int32_t group;
  int32_t pad;
  int64_t kbeg;
  int64_t kend;
  float* o;    // [n_q, H, d]
  float* lse;  // [n_q, H]
};

constexpr int kMaxJobs = 32;

struct AttnParams {
  const void* q;
  int64_t q_stride;
  int64_t n_q;
  int32_t H;
  int32_t n_qtiles;
  float c;  // scale * log2(e)
  int32_t n_jobs;
  int32_t n_segs[2];
  AttnSeg segs[2][ISPA_MAX_SEGS];
  AttnJob jobs[kMaxJobs];
  // single-pass dual form (one workgroup per query tile and head over both
  // groups, merged in its epilogue): 16-bit outputs
  void* a_loc;     // [n_q, H, d] of out_dt: the local group's output
  void* delta;     // [n_q, H, d] of out_dt: merged - a_loc
  float* lse_full; // [n_q, H] or null
  int32_t out_dt;  // ISPA_BF16 or ISPA_F16
  float* o_stash;  // fp32 [n_q, H, d]: the local group's unnormalised output, from the boundary to the epilogue
  // per-group form, d = 128 kernel: when set, the job of group 0 (which then
  // covers the whole group) writes its output here as 16-bit rows [n_q, H, d]
  // of o16_dt instead of fp32 rows to its job's o (its LSE as before)
  void* o16;
  int32_t o16_dt;  // ISPA_BF16 or ISPA_F16
};

// A group description on the host.
struct HostGroup {
  const ispa_seg* segs;
  int32_t n_segs;
  int64_t n_keys() const {
    int64_t t = 0;
    for (int i = 0; i < n_segs; ++i) t += segs[i].n;
    return t;
  }
};

// Plan of how a group's keys are cut into jobs.
struct SplitPlan {
  int n_splits[2];
  int64_t split_len[2];
};

// Queries per workgroup of the kernel that runs (dtype, head_dim).
int attn_block_q(ispa_dtype dt, int32_t d);

// Choose splits so the launch has enough equal-sized work units.
SplitPlan plan_splits(int bq, int64_t n_q, int32_t H, const HostGroup* groups, int n_groups,
                      int max_jobs = kMaxJobs);

// Workspace bytes for the partial (o, lse) of the split groups.
size_t split_workspace_bytes(int64_t n_q, int32_t H, int32_t d, const SplitPlan& plan, int n_groups);
// Partials of every group, split or not (the merged mode of run_group_attention).
size_t merged_workspace_bytes(int64_t n_q, int32_t H, int32_t d, const SplitPlan& plan, int n_groups);

// Run attention for n_groups (1 or 2) groups.  For each group the final
// normalised o / lse go to o_out[g] / lse_out[g]; split groups use ws for
// partials and are merged with the LSE rule.
struct MergeOut;
// With o16_g0 set, group 0's output is (also) written there as 16-bit o16_dt;
// when group 0 is split into merged parts, that replaces its fp32 output.
ispa_status run_group_attention(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, float scale,
                                const void* q, int64_t q_stride, const HostGroup* groups,
                                int n_groups, float* const* o_out, float* const* lse_out,
                                void* ws, size_t ws_bytes, hipStream_t stream,
                                void* o16_g0 = nullptr, int o16_dt = ISPA_BF16,
                                const MergeOut* merge_all = nullptr);

// The single-pass dual form applies (bf16 inputs, d = 128, 16-bit outputs,
// at most 4 runs of rows over both groups, enough (query tile, head) pairs
// to fill the chip): ispa_dual_attn_merge then needs no workspace.
bool dual_single_pass(ispa_dtype dt, int64_t n_q, int32_t H, int32_t d, const HostGroup* groups, int out_dt);
// ws: n_q * H * d fp32 (the local output between the group boundary and the epilogue)
ispa_status run_dual_single_pass(int64_t n_q, int32_t H, float scale, const void* q, int64_t q_stride,
                                 const HostGroup* groups, void* a_loc, void* delta, int out_dt, float* lse_full,
                                 void* ws, hipStream_t stream);

// n-way merge used both by the public call and by split combining.
struct MergeParams {
  int32_t n_parts;
  int32_t d;
  int64_t n_rows;  // n_q * H
  const float* o[16];
  const float* lse[16];
  float* o_full;
  float* lse_full;
  void* a0;
  void* delta;
  int32_t out_dt;
  void* o16;       // optional: the merged output again, as 16-bit o16_dt
  int32_t o16_dt;
  int32_t n_first;  // a0 and delta refer to the merge of parts [0, n_first) (0 means 1)
};

// All groups' parts merged in one pass (run_group_attention): a0 = the merged
// first group, delta = merge of everything - a0, both as out_dt; lse_full the
// merged LSE (optional).
struct MergeOut {
  void* a0;
  void* delta;
  int32_t out_dt;
  float* lse_full;
};
ispa_status launch_merge(const MergeParams& p, hipStream_t stream);

}  // namespace ispa
