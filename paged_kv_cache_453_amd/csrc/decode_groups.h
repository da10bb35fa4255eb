// Sharing groups of a decode batch, as both decode passes read them (device
// side; the host entry point is pa_decode_shared_prefix).
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// Grouped pass over shared prefixes.  Samples of one prompt keep its blocks in
// common ("vLLM 基本原理", section 内存共享), as do requests that hit one cached
// prefix (xdnf.cn article, section 六.3); their block tables then name the same
// physical blocks, and a partition made of such blocks holds the same K/V for
// every sharer.  The grouped pass streams each such partition once and scores
// it against the queries of up to group_members sharers at a time, writing
// each sharer's partial (o_p, lse_p) exactly where its own split-K workgroup
// would have; the regular pass then skips those partitions.
//
// grouped_parts(s): how many leading partitions of sequence s the grouped pass
// computes -- those inside the full blocks that s and its group's leader both
// declare shared.  Both passes evaluate it from the same data, so every
// partition is computed exactly once.  It is 0 (the regular pass does all)
// unless s's group is well formed: leader <= s, the leader leads itself, and
// the first member of s's window of group_members is in the group too, and
// both lengths are within the call's limits.
__device__ __forceinline__ int grouped_parts(const DecodeArgs& a, int s) {
  if (a.prefix_group == nullptr) return 0;
  const int lead = a.prefix_group[s];
  if (lead < 0 || lead > s) return 0;
  const int M = a.group_members;
  const int first = lead + (s - lead) / M * M;
  if (a.prefix_group[lead] != lead || a.prefix_group[first] != lead) return 0;
  const int cap = min(a.max_context_len, a.max_blocks_per_seq * kBlock);
  const int ls = a.context_lens[s];
  const int ll = a.context_lens[lead];
  if (ls < 0 || ll < 0 || ls > cap || ll > cap) return 0;
  const int nb = min(min(a.shared_prefix_blocks[s], a.shared_prefix_blocks[lead]),
                     min(ls, ll) / kBlock);
  return nb > 0 ? nb / a.partition_blocks : 0;
}

// Window size for a launch: at most `slots` query slots (members x query heads
// per kv head) per workgroup; 0 (no grouped pass) when fewer than two members
// fit or the call has no groups.
inline int group_window(const DecodeArgs& a, int slots) {
  if (a.prefix_group == nullptr || a.group <= 0) return 0;
  const int m = a.group_members < slots / a.group ? a.group_members : slots / a.group;
  return m >= 2 ? m : 0;
}

}  // namespace pa
