// Partitioning constants shared by the attention launcher and the host work
// planner: one main-kernel work item covers one partition of a sequence for one
// KV head.
#pragma once

namespace pkv {

constexpr int kDefaultPartition = 512;   // tokens per partition when the caller passes 0
constexpr int kMaxPartitionBlocks = 128;  // a partition spans at most 128 blocks (two per lane)

// Partition size the call resolves to, or 0 when partition_size is not a positive
// multiple of 32 and of B spanning at most kMaxPartitionBlocks blocks (0 = default).
inline int resolve_partition(int partition_size, int B) {
  const int P = partition_size > 0 ? partition_size : kDefaultPartition;
  if (partition_size < 0 || B <= 0 || P % 32 != 0 || P % B != 0 || P / B > kMaxPartitionBlocks)
    return 0;
  return P;
}

}  // namespace pkv
