// C ABI of the paged decode-attention library: argument checks, the launch
// plan (scheduling mode, work-group size, workspace) and dispatch.
// Everything here is host code; it never reads device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/paged_attn.h"
#include "pa_internal.h"

namespace {

constexpr int kDefaultPrefetch = PA_PREFETCH_REG;
constexpr int kMaxPartitionBlocks = 1024;  // LDS slice of the block table: 4 KiB

// What the plan needs to know of the device: the CUs the grid is spread
// over and the LDS a CU and a work-group can hold.  Queried once per device
// (hipDeviceGetAttribute) and cached; where no device can be queried the
// MI355X figures stand in (256 CUs, 160 KiB of LDS per CU and per
// work-group).
struct DeviceInfo {
  int64_t cus;
  size_t lds_per_cu;
  size_t lds_per_wg;
};
constexpr DeviceInfo kMI355X = {256, 163840, 163840};

// Auto plan, from measurements over the model shapes, their tensor-parallel
// shards and a batch x context grid (U = sequences x KV heads, C = CUs):
//  * U >= C (one work-group per CU): no split, so no partials and no reduce
//    launch.  Splitting further only added per-partition overhead, even for
//    ragged batches once the longest sequences are dispatched first.
//  * Such work-groups get 8 waves while U < kFourWaveUnitsPerCU * C and the
//    table is at least kLongTableBlocks wide: with under three work-groups
//    per CU the long sequences then finish on twice the waves (up to 9 % on
//    a ragged batch, within 2 % either way on uniform ones).  Otherwise 4
//    waves: at 3 resident waves per SIMD a CU holds three 4-wave
//    work-groups but only one 8-wave one.
//  * U < C: about C / U partitions of kMinAutoPartition..kMaxAutoPartition
//    blocks, 8 waves (equal or better than 4 on every split plan measured).
//    Partitions may shrink to kMinShortPartition blocks while that gives at
//    most kReducePartitions of them (the reduce then loads every partial at
//    once): batch 8 x 1K tokens of a GQA 32/8 layer, 34 MB, took 12.9 us as
//    one partition and 9.9 us as four 16-block ones.  Beyond that many
//    partitions the reduce costs more than the extra CUs bring (two
//    64K-token sequences: 37 us in 64-block partitions, 52 us in 32-block
//    ones).
constexpr int64_t kFourWaveUnitsPerCU = 3;
constexpr int kLongTableBlocks = 512;
constexpr int kMinAutoPartition = pa::kReduceBigPartition;
constexpr int kMinShortPartition = 16;
constexpr int kReducePartitions = pa::kReduceRegs;
constexpr int kMaxAutoPartition = 256;
constexpr int kTwoLoopPartitionBlocks = 32;
//  * Auto order ranks the sequences (longest first) only when the grid is
//    larger than what the CUs hold at once.  When every work-group is
//    resident from the start the dispatch order changes nothing, and the
//    ranking (a dependent read of every context length before the block
//    table) only adds latency: 2-4 us on grids of 256 work-groups.
//    Residency: C x min(kResidentWavesPerCU / W, LDS per CU / LDS per
//    work-group); 3 waves per SIMD (of the 4 of a CDNA CU) is what the
//    register ring's VGPRs allow.
constexpr int kResidentWavesPerCU = 12;
//  * The streaming shape, for batches whose contexts all fill the table
//    (pa_options.min_context_hint >= 7/8 of its width) with a whole number u
//    of units per CU and one partition per unit.  A CU streams best with
//    about 32 KiB of K/V loads in flight: 4 fp16 blocks of one KV head (K
//    and V, 8 KiB each), 8 E4M3 ones.  The shapes above keep 8-24 blocks in
//    flight and over-subscribe it by 2-6 %.  The streaming shape picks the
//    waves per work-group and a residency cap from u and from the blocks
//    each wave keeps in flight (1 with the look-ahead off, 2 with the
//    register look-ahead one block ahead, 3 two blocks ahead), so that every
//    CU holds about that many from the start to the end of the launch
//    (stream_shape below).  Measured, us (default shape -> streaming shape,
//    look-ahead on): MHA 32/32, 32 x 2K (llama2_7b-shaped) 159.5 -> 152.8;
//    8 x 4K 79.9 -> 75.7; 16 x 2K 82.1 -> 79.3; 24 x 2K 120.1 -> 117.2;
//    32 x 16K 1253 -> 1208; GQA 32/8, 64 x 16K 627 -> 615; GQA 28/4, 128 x
//    4K 160.2 -> 158.4; GQA 40/8, 128 x 8K 628.6 -> 619.8; E4M3 MHA 32 x 2K
//    81.7 -> 78.6.  With the look-ahead off, 32 x 2K: 161.1 -> 149.9.  Where
//    it did not pay it is left out: other u (a partial last round leaves CUs
//    with one work-group and too few loads in flight; 8 units per CU lost up
//    to 4 % on GQA batches), GQA tables under kStreamMinBlocksGqa blocks
//    (their longer prologue and merge: GQA 32/8 32 x 1K 21.5 -> 22.7), and
//    tables split into partitions.  A ragged batch must not take this
//    shape: its long units then run alone on their CUs with 1-2 blocks in
//    flight (llama3_8b-shaped, 64 x 512..8K tokens: 181 -> 256 us), hence
//    the hint.
constexpr int kStreamMinBlocks = 64;
// The largest residency cap the LDS request enforces on 160 KiB of LDS per
// CU: beyond about 10 the 1 KiB margin for the compiler's LDS and the
// allocation granularity is a large part of each work-group's share.
constexpr int kMaxResidencyCap = 8;
constexpr int kStreamMinBlocksGqa = 256;
constexpr int kStreamSplitBlocks = 256;
// The even split's shortest table (blocks) for the auto plan.
constexpr int kEvenMinBlocks = 160;
// What a piece change costs a share, in blocks read: the shares are cut as
// if every (sequence, KV head) unit began with this many more blocks, so a
// share that crosses more unit starts gets fewer blocks.  A share's end time
// grew about 3 us per piece on the llama3_8b TP2 shard, where a CU reads an
// 8 KiB fp16 block (4 KiB E4M3) in about 0.3 us (0.15 us); swept over
// 0..20 (fp16) and 10..30 (E4M3) on five ragged batches, 12 and 20..30 were
// the fastest (12 against 10: 0.2-0.5 us).
constexpr int kEvenPieceBlocksF16 = 12;
constexpr int kEvenPieceBlocksE4M3 = 24;

bool valid_device(const pa_device_info* d) {
  return d && d->compute_units >= 1 && d->compute_units <= 65536 &&
         d->lds_bytes_per_workgroup >= 1024 &&
         d->lds_bytes_per_cu >= d->lds_bytes_per_workgroup;
}

DeviceInfo from_public(const pa_device_info* d) {
  return DeviceInfo{d->compute_units, (size_t)d->lds_bytes_per_cu,
                    (size_t)d->lds_bytes_per_workgroup};
}

// The current device's figures, cached per device; the MI355X figures (and
// queried = 0) when there is no device to query.
void current_device(pa_device_info* out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static pa_device_info cache[kMaxDevices];
  static bool have[kMaxDevices];
  out->compute_units = (int32_t)kMI355X.cus;
  out->lds_bytes_per_cu = (int32_t)kMI355X.lds_per_cu;
  out->lds_bytes_per_workgroup = (int32_t)kMI355X.lds_per_wg;
  out->queried = 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    int cus = 0, lds_cu = 0, lds_wg = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&lds_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess)
      return;
    pa_device_info q;
    q.compute_units = cus;
    q.lds_bytes_per_workgroup = lds_wg;
    q.lds_bytes_per_cu = lds_cu > lds_wg ? lds_cu : lds_wg;
    q.queried = 1;
    if (!valid_device(&q)) return;
    cache[dev] = q;
    have[dev] = true;
  }
  *out = cache[dev];
}

DeviceInfo current_device_info() {
  pa_device_info d;
  current_device(&d);
  return from_public(&d);
}

struct Plan {
  int pf, dist, waves, PB, P, order, two;
  int64_t wgs;
  size_t ws_bytes;
  int bal, nslot, pb_max;  // balanced split: grid rows per KV head, largest size
  int cap;                 // residency cap (work-groups per CU), 0 = none
  size_t lds;              // dynamic LDS per decode work-group
  int chain;               // sequences one work-group walks in turn (1 or 2)
  int even;                // 1: the even split over `wgs` shares
};

// Waves per work-group and residency cap of the streaming shape for u units
// per CU, by the blocks `f` each wave keeps in flight ({0, 0} where it does
// not apply: other u, the L2 touch, the LDS ring).
struct StreamShape {
  int waves, cap;
};
StreamShape stream_shape(int64_t u, bool kv8, int f) {
  if (kv8) {  // 8 blocks of 4 KiB
    if (f == 1 && u == 1) return {8, 0};
    if (f == 1 && u == 4) return {2, 4};
    if (f == 3 && u == 4) return {1, 4};
    return {0, 0};
  }
  if (f == 1) {  // 4 blocks of 8 KiB: 4 waves per CU
    switch (u) {
      case 1: return {4, 0};
      case 2: return {2, 0};
      case 3: return {4, 1};
      case 4: return {1, 4};
      case 6: return {2, 2};
      default: return {0, 0};
    }
  }
  if (f == 2) {  // 2 waves per CU
    switch (u) {
      case 1: return {2, 0};
      case 2: return {1, 0};
      case 3: return {2, 1};
      case 4: case 6: return {1, 2};
      default: return {0, 0};
    }
  }
  return {0, 0};
}

// Balanced split (auto partitions of a ragged batch with fewer (sequence,
// KV head) pairs than CUs, 2..PA_RANK_MAX_SEQS sequences): the device picks
// the partition size from the context lengths so that each KV head's
// partitions fill about one work-group per CU; sizes are multiples of the
// wave count from kMinShortPartition blocks up.  On uniform batches it
// makes the same partitions as the fixed rule; on llama3_8b-shaped TP
// shards the longest sequences no longer run alone on their CUs.
constexpr int kBalancedMaxTable = 65536;  // blocks; keeps the device's float division exact

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(const pa_shape* sh) {
  if (!sh) return PA_ERR_INVALID_ARG;
  if (sh->num_seqs < 1 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 ||
      sh->max_blocks_per_seq < 1 || sh->num_blocks < 1)
    return PA_ERR_INVALID_ARG;
  if (sh->num_q_heads % sh->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (sh->head_dim != PA_HEAD_DIM || sh->block_size != PA_BLOCK_SIZE)
    return PA_ERR_UNSUPPORTED;
  const int g = sh->num_q_heads / sh->num_kv_heads;
  if (g > PA_G_MAX) return PA_ERR_UNSUPPORTED;
  // grid.x = Hkv and grid.y = B must fit the launch limits.
  if (sh->num_kv_heads > 65535 || sh->num_seqs > 65535) return PA_ERR_UNSUPPORTED;
  // Byte offsets of the pool and token counts must fit their types.
  if (sh->num_blocks > (INT64_MAX / 8192) / sh->num_kv_heads) return PA_ERR_UNSUPPORTED;
  const int64_t strides[4] = {sh->k_block_stride, sh->k_head_stride, sh->v_block_stride,
                              sh->v_head_stride};
  for (int64_t st : strides) {
    if (st < 0 || (st & 15)) return PA_ERR_INVALID_ARG;
    if (st > 0 && st > INT64_MAX / 4 / sh->num_blocks) return PA_ERR_UNSUPPORTED;
  }
  if (sh->max_blocks_per_seq > INT32_MAX / PA_BLOCK_SIZE) return PA_ERR_UNSUPPORTED;
  if (sh->kv_dtype != PA_KV_F16 && sh->kv_dtype != PA_KV_E4M3) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int make_plan(const pa_shape* sh, const pa_options* o, const DeviceInfo& dv, Plan* pl) {
  int rc = check_shape(sh);
  if (rc) return rc;
  pa_options d;
  paged_attn_default_options(&d);
  if (!o) o = &d;
  if (o->prefetch_distance < 0 || o->prefetch_distance > 63) return PA_ERR_INVALID_ARG;
  if (o->structure != PA_STRUCTURE_FUSED && o->structure != PA_STRUCTURE_TWO_LOOP)
    return PA_ERR_INVALID_ARG;
  const bool two = o->structure == PA_STRUCTURE_TWO_LOOP;
  const bool kv8 = sh->kv_dtype == PA_KV_E4M3;
  if (two && (o->prefetch_distance > 1 || kv8)) return PA_ERR_UNSUPPORTED;
  if (o->min_context_hint < 0 || o->max_resident_wgs < 0 ||
      o->max_resident_wgs > kMaxResidencyCap)
    return PA_ERR_INVALID_ARG;
  int order = o->seq_order;
  if (order < PA_ORDER_AUTO || order > PA_ORDER_LONGEST_FIRST) return PA_ERR_INVALID_ARG;
  if (order == PA_ORDER_AUTO)
    order = sh->num_seqs >= 2 && sh->num_seqs <= PA_RANK_MAX_SEQS ? PA_ORDER_LONGEST_FIRST
                                                                  : PA_ORDER_NATURAL;
  if (order == PA_ORDER_LONGEST_FIRST && sh->num_seqs > PA_RANK_MAX_SEQS)
    return PA_ERR_UNSUPPORTED;
  const int g = sh->num_q_heads / sh->num_kv_heads;

  int pf = o->prefetch < 0 ? kDefaultPrefetch : o->prefetch;
  if (pf > PA_PREFETCH_LDS) return PA_ERR_INVALID_ARG;
  // Default distance 1, except the register and LDS look-aheads over an E4M3
  // cache: its blocks are half the bytes, and two of them ahead (at 142
  // VGPRs, still 3 waves per SIMD, for the registers) measured up to 10 %
  // faster on a ragged batch.
  const bool ring = pf == PA_PREFETCH_REG || pf == PA_PREFETCH_LDS;
  int dist = o->prefetch_distance > 0 ? o->prefetch_distance : (kv8 && ring ? 2 : 1);
  // the register and LDS rings hold at most two blocks ahead
  if (ring && dist > 2) return PA_ERR_UNSUPPORTED;
  if (pf == PA_PREFETCH_LDS && two) return PA_ERR_UNSUPPORTED;
  // the LDS ring: dist + 1 slots of one block's K and V per wave
  const size_t slot = pf == PA_PREFETCH_LDS
                          ? (size_t)(dist + 1) * 2 * PA_BLOCK_SIZE * PA_HEAD_DIM * (kv8 ? 1 : 2)
                          : 0;

  const int B = sh->num_seqs, Hkv = sh->num_kv_heads;
  const int MB = sh->max_blocks_per_seq;
  const int64_t units = (int64_t)B * Hkv;
  bool rank = order == PA_ORDER_LONGEST_FIRST;
  if (o->waves_per_wg != 0 && o->waves_per_wg != 1 && o->waves_per_wg != 2 &&
      o->waves_per_wg != 4 && o->waves_per_wg != 8)
    return PA_ERR_INVALID_ARG;
  if (o->partition_blocks < 0) return PA_ERR_INVALID_ARG;
  if (o->partition_blocks > kMaxPartitionBlocks) return PA_ERR_UNSUPPORTED;

  int waves = o->waves_per_wg;
  int cap = o->max_resident_wgs;
  // the streaming shape: every context at least 7/8 of the table, a whole
  // number of units per CU, the look-ahead off or in registers (the
  // measured distances), waves, partitions and residency left to the plan
  const int in_flight = pf == PA_PREFETCH_OFF ? 1 : pf == PA_PREFETCH_REG ? 1 + dist : 0;
  const bool streaming = o->min_context_hint > 0 &&
                         (int64_t)o->min_context_hint * 8 >= (int64_t)MB * PA_BLOCK_SIZE * 7 &&
                         MB >= (g == 1 ? kStreamMinBlocks : kStreamMinBlocksGqa) && !two &&
                         in_flight > 0 && o->waves_per_wg == 0 && o->partition_blocks == 0 &&
                         o->max_resident_wgs == 0;
  if (streaming && units >= dv.cus && units % dv.cus == 0 && MB <= kMaxPartitionBlocks) {
    const StreamShape ss = stream_shape(units / dv.cus, kv8, in_flight);
    if (ss.waves > 0) {
      waves = ss.waves;
      cap = ss.cap;
      // uniform contexts: the ranking would be the identity
      if (o->seq_order == PA_ORDER_AUTO) {
        order = PA_ORDER_NATURAL;
        rank = false;
      }
    }
  }
  // Fewer units than CUs, split by the balanced rule into about one
  // work-group per CU: with at least kStreamSplitBlocks blocks per CU, the
  // same 4 fp16 blocks in flight (2 waves one block ahead, or 4 without the
  // look-ahead) beat the 8 waves of the split plans by 0.5-2 % (us, 8 waves
  // -> 2: GQA 32/8 8 x 32K 164.5 -> 161.6, 16 x 16K 164.9 -> 161.7, 16 x
  // 8K 83.9 -> 83.4; GQA 5/1 128 x 8K 85.9 -> 84.8); on shorter walks the
  // 8 waves hide more of the start-up (GQA 32/8 16 x 4K: 45.1 against 45.5).
  if (streaming && !kv8 && units < dv.cus && o->seq_order == PA_ORDER_AUTO && B >= 2 &&
      B <= PA_RANK_MAX_SEQS && MB <= kBalancedMaxTable &&
      (int64_t)MB * units >= (int64_t)kStreamSplitBlocks * dv.cus && in_flight <= 2)
    waves = in_flight == 1 ? 4 : 2;
  // The even split (pa_options.even_split): one share of the batch's
  // blocks per work-group, S = CUs x the residency cap (1 unless asked).
  //
  // The plan takes it by itself for a batch of 2..256 sequences with at
  // least C / 2 units and 160..1024 table blocks, unless the hint says every
  // context fills the table (a uniform batch takes the streaming shape,
  // which is faster).  The fixed grid leaves CUs idle on a ragged batch (a
  // last round of fewer units than CUs, or long units alone on their CUs)
  // and the balanced split keeps partitions of one size.  Measured (us, the
  // plan before -> the even split, with the piece charge): llama3_8b (64 x
  // 512..8K, 512 units) 181.4 -> 175.3; its TP2 shard 106.0 -> 93.3, TP4
  // shard 53.3 -> 50.5; GQA 32/8 96 x 512..8K 299.0 -> 260.2, 64 x 1..8K
  // 199.9 -> 168.7, 256 x 1..4K 347.2 -> 334.2; GQA 40/8 48 x 1..8K 175.5
  // -> 130.8;
  // E4M3 llama3_8b TP2 59.5 -> 51.0, TP4 32.7 -> 29.1, llama3_8b 96.2 ->
  // 96.3; tables of 160..223 blocks 0.5-11 % faster (GQA 32/8 64 x 1..3K
  // 76.8 -> 70.2).  It lost on shorter tables (GQA 32 x 1..2K, 128 blocks:
  // 27.5 -> 29.7; 64 blocks: 13-16 %), below C / 2 units in fp16 (the TP8
  // shard 28.6 -> 29.4) and on uniform batches planned without the hint
  // (qwen25_7b 158.4 -> 163.5).  E4M3 also takes it from C / 4 units with
  // groups of at most 8 query heads: 4-8 % faster there (the llama3_8b TP8
  // shard 19.1 -> 18.3; GQA 4/1 96 x 512..8K 25.4 -> 23.5), but 6 % slower
  // with 16 (GQA 32/2 32 x 512..8K 21.5 -> 22.9).
  if (o->even_split < PA_EVEN_SPLIT_AUTO || o->even_split > PA_EVEN_SPLIT_ON)
    return PA_ERR_INVALID_ARG;
  const bool uniform_hint = o->min_context_hint > 0 && (int64_t)o->min_context_hint * 8 >=
                                                           (int64_t)MB * PA_BLOCK_SIZE * 7;
  const bool even_auto =
      o->even_split == PA_EVEN_SPLIT_AUTO && !two && !uniform_hint && in_flight > 0 &&
      o->partition_blocks == 0 && o->waves_per_wg == 0 && o->max_resident_wgs == 0 &&
      o->seq_order == PA_ORDER_AUTO && B >= 2 && B <= PA_RANK_MAX_SEQS &&
      MB >= kEvenMinBlocks && MB <= kMaxPartitionBlocks &&
      (2 * units >= dv.cus || (kv8 && g <= 8 && 4 * units >= dv.cus)) &&
      (int64_t)B * (MB + kEvenPieceBlocksE4M3) * Hkv <= INT32_MAX / 2;
  const bool even = o->even_split == PA_EVEN_SPLIT_ON || even_auto;
  if (even) {
    // positions in the (block, KV head) sequence are int32 on the device
    if (two || o->partition_blocks != 0 || B > PA_RANK_MAX_SEQS || MB > kMaxPartitionBlocks ||
        (int64_t)B * (MB + kEvenPieceBlocksE4M3) * Hkv > INT32_MAX / 2)
      return PA_ERR_UNSUPPORTED;
    // fp16: 2 waves one block ahead, or 4 without the look-ahead (4 blocks
    // per work-group); E4M3: 8 waves, the register look-ahead one block
    // ahead unless asked (us, over 2 ahead or 2-4 waves: llama3_8b TP2
    // 55.5 -> 53.9, 48 x 1..8K 77.4 -> 74.8, 32 x 512..8K 55.9 -> 54.1)
    if (kv8 && pf == PA_PREFETCH_REG && o->prefetch_distance == 0) dist = 1;
    waves = o->waves_per_wg;
    if (waves == 0) waves = kv8 ? 8 : in_flight == 1 ? 4 : 2;
    cap = o->max_resident_wgs > 0 ? o->max_resident_wgs : 1;
    order = PA_ORDER_NATURAL;
    rank = false;
  }
  if (waves == 0 && two) waves = 4;
  if (waves == 0) {
    const bool whole = o->partition_blocks == 0 ? units >= dv.cus : o->partition_blocks >= MB;
    waves = 4;
    if (whole && units < kFourWaveUnitsPerCU * dv.cus && MB >= kLongTableBlocks &&
        MB <= kMaxPartitionBlocks &&
        pa::decode_lds_bytes(MB, g, 8, B, rank, 8 * slot) + pa::kCompilerLdsBytes <=
            dv.lds_per_wg)
      waves = 8;
    const int split_pb = MB < kMaxAutoPartition ? MB : kMaxAutoPartition;
    if (o->partition_blocks == 0 && !whole &&
        pa::decode_lds_bytes(split_pb, g, 8, B, rank, 8 * slot) + pa::kCompilerLdsBytes <=
            dv.lds_per_wg)
      waves = 8;
  }

  int PB;
  if (even) {
    PB = MB;  // a piece is at most one sequence's table
  } else if (o->partition_blocks > 0) {
    PB = o->partition_blocks < MB ? o->partition_blocks : MB;
  } else if (two) {
    // 512-token partitions, halved until the scores fit in LDS
    PB = kTwoLoopPartitionBlocks < MB ? kTwoLoopPartitionBlocks : MB;
    while (PB > 1 && pa::two_loop_lds_bytes(PB, g, waves, B, rank) + pa::kCompilerLdsBytes >
                          dv.lds_per_wg)
      PB /= 2;
  } else if (units >= dv.cus) {
    PB = MB < kMaxPartitionBlocks ? MB : kMaxPartitionBlocks;
  } else {
    const int64_t want = (dv.cus + units - 1) / units;
    int64_t pb = (MB + want - 1) / want;
    pb = (pb + waves - 1) / waves * waves;  // whole rounds of the W waves
    if (pb < kMinAutoPartition) {
      const int64_t shortest = pb > kMinShortPartition ? pb : kMinShortPartition;
      pb = (MB + shortest - 1) / shortest <= kReducePartitions ? shortest : kMinAutoPartition;
    }
    if (pb > kMaxAutoPartition) pb = kMaxAutoPartition;
    if (pb > MB) pb = MB;
    PB = (int)pb;
  }
  int P = (MB + PB - 1) / PB;
  if (P > 65535) return PA_ERR_UNSUPPORTED;  // grid.z
  // the balanced split replaces the fixed partitions of an auto split plan
  int bal = 0, nslot = 0, pb_max = 0;
  if (!even && !two && o->partition_blocks == 0 && units < dv.cus &&
      o->seq_order == PA_ORDER_AUTO && B >= 2 && B <= PA_RANK_MAX_SEQS &&
      MB <= kBalancedMaxTable) {
    const int pb_min = (kMinShortPartition + waves - 1) / waves * waves;
    const int cap = MB < kMaxPartitionBlocks ? MB : kMaxPartitionBlocks;
    pb_max = (cap + waves - 1) / waves * waves;
    if (pb_max < pb_min) pb_max = pb_min;
    // rows per KV head: one work-group per CU, and at least what the
    // largest size needs in the worst case
    const int64_t need = (int64_t)B * ((MB + pb_max - 1) / pb_max);
    const int64_t rows = dv.cus / Hkv > need ? dv.cus / Hkv : need;
    // partitions one sequence can get: its table in partitions of the
    // smallest size, at most kReducePartitions of them unless they hold at
    // least kMinAutoPartition blocks (the device keeps both rules), and at
    // most rows - B + 1
    int64_t per_seq = (MB + pb_min - 1) / pb_min;
    const int64_t big = (MB + kMinAutoPartition - 1) / kMinAutoPartition;
    const int64_t red = big > kReducePartitions ? big : kReducePartitions;
    per_seq = per_seq < red ? per_seq : red;
    const int64_t most = rows - B + 1;
    if (rows <= 65535 && per_seq > 1) {  // one partition per sequence needs no split
      bal = 1;
      nslot = (int)rows;
      PB = pb_min;
      P = (int)(per_seq < most ? per_seq : most);
      order = PA_ORDER_NATURAL;
      rank = false;
    }
  }
  auto lds_for = [&](bool r) {
    return two ? pa::two_loop_lds_bytes(PB, g, waves, B, r)
               : pa::decode_lds_bytes(bal ? pb_max : PB, g, waves, B, r, waves * slot);
  };
  // Two sequences per work-group, in turn: 1-wave work-groups capped at 2
  // per CU hand a CU over to a new work-group twice per round, and each
  // handover (the finished wave's output, the next one's context length,
  // table slice and first loads) leaves the CU with half its loads in
  // flight for a few us.  A wave that walks two sequences skips the
  // dispatch between them; grid row y takes sequence ranks y and B-1-y, so
  // under longest-first order a long sequence pairs with a short one.  Only
  // where the halved grid still fills whole rounds of the cap (MHA 32/32, 32
  // x 2K: 152.4 -> 150.9 us).
  int chain = 1;
  if (!even && !two && !bal && P == 1 && waves == 1 && cap == 2 && B % 2 == 0 &&
      units % ((int64_t)2 * cap * dv.cus) == 0)
    chain = 2;
  const int64_t wgs = even  ? (int64_t)dv.cus * cap
                      : bal ? (int64_t)nslot * Hkv
                            : (int64_t)P * Hkv * B / chain;
  // a residency cap takes LDS: cap work-groups of it fill a CU
  const size_t cap_lds = cap > 0 ? pa::residency_lds_bytes(dv.lds_per_cu, cap) : 0;
  auto lds_with_cap = [&](bool r) {
    const size_t l = lds_for(r);
    return l > cap_lds ? l : cap_lds;
  };
  if (o->seq_order == PA_ORDER_AUTO && rank) {
    const size_t l = lds_with_cap(true) + pa::kCompilerLdsBytes;
    const int64_t by_waves = kResidentWavesPerCU / waves;
    const int64_t by_lds = (int64_t)(dv.lds_per_cu / l);
    if (wgs <= dv.cus * (by_waves < by_lds ? by_waves : by_lds)) {
      order = PA_ORDER_NATURAL;
      rank = false;
    }
  }
  const size_t lds = lds_with_cap(rank);
  if (lds + pa::kCompilerLdsBytes > dv.lds_per_wg) return PA_ERR_UNSUPPORTED;
  memset(pl, 0, sizeof(*pl));
  pl->order = order;
  pl->two = two ? 1 : 0;
  pl->pf = pf;
  pl->dist = dist;
  pl->waves = waves;
  pl->PB = PB;
  pl->P = P;
  pl->wgs = wgs;
  pl->bal = bal;
  pl->nslot = nslot;
  pl->pb_max = pb_max;
  pl->cap = cap;
  pl->chain = chain;
  pl->even = even ? 1 : 0;
  pl->lds = lds;
  // partials [B][Hq][P][128] and [B][Hq][P][2] in fp32; the balanced split
  // adds the sequences' partition counts (B int32, padded to 16 bytes)
  pl->ws_bytes = P > 1 ? ((size_t)(bal ? (B + 3) / 4 * 4 : 0) +
                          (size_t)B * sh->num_q_heads * P * (2 + PA_HEAD_DIM)) *
                             sizeof(float)
                       : 0;
  // the even split: two records of g rows (128 outputs, then m and l) per
  // share, then (first record, pieces) per (sequence, KV head)
  if (even) pl->ws_bytes = (pa::even_records(wgs, g) + (size_t)2 * units) * sizeof(float);
  return PA_OK;
}

}  // namespace

extern "C" {

void paged_attn_default_options(pa_options* o) {
  if (!o) return;
  memset(o, 0, sizeof(*o));
  o->prefetch = -1;
}

int paged_attn_device_info(pa_device_info* info) {
  if (!info) return PA_ERR_INVALID_ARG;
  current_device(info);
  return PA_OK;
}

static int plan_info(const pa_shape* sh, const pa_options* o, const DeviceInfo& dv,
                     pa_plan_info* info) {
  if (!info) return PA_ERR_INVALID_ARG;
  Plan pl;
  int rc = make_plan(sh, o, dv, &pl);
  if (rc) return rc;
  memset(info, 0, sizeof(*info));
  info->prefetch = pl.pf;
  info->waves_per_wg = pl.waves;
  info->partition_blocks = pl.PB;
  info->num_partitions = pl.P;
  info->workgroups = pl.wgs;
  info->workspace_bytes = pl.ws_bytes;
  info->seq_order = pl.order;
  info->structure = pl.two;
  info->prefetch_distance = pl.dist;
  info->balanced = pl.bal;
  info->resident_wgs = pl.cap;
  info->lds_bytes = pl.lds;
  info->seqs_per_wg = pl.chain;
  info->even_split = pl.even;
  return PA_OK;
}

int paged_attn_plan(const pa_shape* sh, const pa_options* o, pa_plan_info* info) {
  return plan_info(sh, o, current_device_info(), info);
}

int paged_attn_plan_for_device(const pa_shape* sh, const pa_options* o,
                               const pa_device_info* dev, pa_plan_info* info) {
  if (!valid_device(dev)) return PA_ERR_INVALID_ARG;
  return plan_info(sh, o, from_public(dev), info);
}

size_t paged_attn_workspace_size(const pa_shape* sh, const pa_options* o) {
  Plan pl;
  if (make_plan(sh, o, current_device_info(), &pl)) return 0;
  return pl.ws_bytes;
}

}  // extern "C"

namespace {

// Checks of the tensor pointers and scalars of a decode call.
int check_args(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, const int32_t* context_lens, float scale, bool kv8,
               float k_scale, float v_scale, const void* out, const pa_shape* sh) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return PA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
      (reinterpret_cast<uintptr_t>(context_lens) & 3u))
    return PA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (!isfinite(k_scale) || !isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return PA_ERR_INVALID_ARG;
  if (sh && sh->kv_dtype != (kv8 ? PA_KV_E4M3 : PA_KV_F16)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Shared by the fp16 and the E4M3 entry points.
int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, float scale,
                bool kv8, float k_scale, float v_scale, void* out, const pa_shape* sh,
                const pa_options* o, void* stream) {
  int rc = check_args(q, k_cache, v_cache, block_tables, context_lens, scale, kv8, k_scale,
                      v_scale, out, sh);
  if (rc) return rc;
  Plan pl;
  rc = make_plan(sh, o, current_device_info(), &pl);
  if (rc) return rc;
  // cache strides: 0 = dense; slices may be spread out but never overlap
  const int64_t slice = (int64_t)PA_BLOCK_SIZE * PA_HEAD_DIM * (kv8 ? 1 : 2);
  const int64_t k_head = sh->k_head_stride ? sh->k_head_stride : slice;
  const int64_t v_head = sh->v_head_stride ? sh->v_head_stride : slice;
  const int64_t k_blk = sh->k_block_stride ? sh->k_block_stride : k_head * sh->num_kv_heads;
  const int64_t v_blk = sh->v_block_stride ? sh->v_block_stride : v_head * sh->num_kv_heads;
  if (k_head < slice || v_head < slice || k_blk < k_head * sh->num_kv_heads ||
      v_blk < v_head * sh->num_kv_heads)
    return PA_ERR_INVALID_ARG;
  pa_options d;
  paged_attn_default_options(&d);
  if (!o) o = &d;
  if (pl.ws_bytes > 0) {
    if (!o->workspace || o->workspace_bytes < pl.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned16(o->workspace)) return PA_ERR_INVALID_ARG;
  }
  if ((o->debug_gather_k && !aligned16(o->debug_gather_k)) ||
      (o->debug_trace && (reinterpret_cast<uintptr_t>(o->debug_trace) & 3u)) ||
      (o->debug_error_word && (reinterpret_cast<uintptr_t>(o->debug_error_word) & 3u)) ||
      (o->debug_timeline && (reinterpret_cast<uintptr_t>(o->debug_timeline) & 7u)))
    return PA_ERR_INVALID_ARG;

  const int g = sh->num_q_heads / sh->num_kv_heads;
  pa::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.q = static_cast<const uint16_t*>(q);
  a.k = k_cache;
  a.v = v_cache;
  a.bt = block_tables;
  a.ctx = context_lens;
  a.out = static_cast<uint16_t*>(out);
  a.dbg_k = static_cast<uint16_t*>(o->debug_gather_k);
  a.dbg_trace = o->debug_trace;
  a.dbg_err = o->debug_error_word;
  a.dbg_timeline = o->debug_timeline;
  a.sink = nullptr;
  a.sink_enable = 0;
  a.rank_seqs = pl.order == PA_ORDER_LONGEST_FIRST ? 1 : 0;
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  a.v_scale = v_scale;
  a.B = sh->num_seqs;
  a.Hq = sh->num_q_heads;
  a.Hkv = sh->num_kv_heads;
  a.G = g;
  a.MB = sh->max_blocks_per_seq;
  a.P = pl.P;
  a.PB = pl.PB;
  a.NB = sh->num_blocks;
  a.k_head = k_head;
  a.v_head = v_head;
  a.k_blk = k_blk;
  a.v_blk = v_blk;
  a.lds_bt_bytes = pa::lds_bt_bytes_for(pl.bal ? pl.pb_max : pl.PB);
  a.balanced = pl.bal;
  a.nslot = pl.nslot;
  a.pb_max = pl.pb_max;
  if (pl.bal) a.k_uniform = pl.nslot / sh->num_seqs < pl.P ? pl.nslot / sh->num_seqs : pl.P;
  a.pf_dist = pl.dist;
  a.chain = pl.chain;
  a.even = pl.even;
  a.shares = pl.even ? (int)pl.wgs : 0;
  a.even_kappa = kv8 ? kEvenPieceBlocksE4M3 : kEvenPieceBlocksF16;
  const bool dbg =
      o->debug_gather_k || o->debug_trace || o->debug_error_word || o->debug_timeline;
  if (pl.two && dbg) return PA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (pl.P > 1) {
    // [rows][128] unnormalised outputs first, so every 512-byte row starts
    // on a cache line, then [rows][2] (m, l), then the balanced split's
    // per-sequence partition counts
    float* ws = static_cast<float*>(o->workspace);
    const size_t rows = (size_t)sh->num_seqs * sh->num_q_heads * pl.P;
    a.ws_o = ws;
    a.ws_ml = ws + rows * PA_HEAD_DIM;
    if (pl.bal) a.ws_np = reinterpret_cast<int32_t*>(a.ws_ml + rows * 2);
  }
  if (pl.even) {
    // [2 S][g][128] outputs, [2 S][g][2] (m, l), then [B][Hkv][2] int32
    float* ws = static_cast<float*>(o->workspace);
    const size_t recs = (size_t)2 * pl.wgs * g;
    a.ws_o = ws;
    a.ws_ml = ws + recs * PA_HEAD_DIM;
    a.ws_np = reinterpret_cast<int32_t*>(ws + pa::even_records(pl.wgs, g));
  }
  if (pl.two) {
    if (pa::launch_decode_two_loop(a, pl.pf, pl.waves, pl.lds, st) != hipSuccess)
      return PA_ERR_HIP;
  } else {
    // the register look-ahead at distance 2 is kernel instance 4, the LDS
    // ring at distance 1 and 2 instances 5 and 6
    const int variant = pl.pf == PA_PREFETCH_LDS ? 4 + pl.dist
                        : pl.pf == PA_PREFETCH_REG && pl.dist == 2 ? 4
                                                                   : pl.pf;
    if (pa::launch_decode(a, variant, dbg, kv8, pl.waves, pl.lds, st) != hipSuccess)
      return PA_ERR_HIP;
  }
  if ((pl.P > 1 || pl.even) && pa::launch_reduce(a, st) != hipSuccess) return PA_ERR_HIP;
  return PA_OK;
}

}  // namespace

extern "C" {

int paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      float scale, void* out, const pa_shape* sh, const pa_options* o,
                      void* stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, false, 1.f, 1.f,
                     out, sh, o, stream);
}

int paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* context_lens,
                          float scale, float k_scale, float v_scale, void* out,
                          const pa_shape* sh, const pa_options* o, void* stream) {
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, true, k_scale,
                     v_scale, out, sh, o, stream);
}

int paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              float scale, void* out, const pa_shape* sh, const pa_options* o,
                              void* stream) {
  int rc = check_args(q, k_cache, v_cache, block_tables, context_lens, scale, false, 1.f, 1.f,
                      out, sh);
  if (rc) return rc;
  pa_options oo;
  if (o) {
    oo = *o;
  } else {
    paged_attn_default_options(&oo);
  }
  Plan pl;
  rc = make_plan(sh, &oo, current_device_info(), &pl);
  if (rc) return rc;
  if (pl.ws_bytes > pa::kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
  // the current device's copy of the library's scratch array (its address
  // is looked up on the first call on each device); nothing is allocated
  void* scratch = nullptr;
  if (pa::noalloc_scratch(&scratch) != hipSuccess) return PA_ERR_HIP;
  oo.workspace = scratch;
  oo.workspace_bytes = pa::kNoAllocScratchBytes;
  return decode_impl(q, k_cache, v_cache, block_tables, context_lens, scale, false, 1.f, 1.f,
                     out, sh, &oo, stream);
}

int paged_attn_pack_k(const void* k_token_major, void* k_cache, int64_t num_blocks,
                      int32_t num_kv_heads, int32_t kv_dtype, void* stream) {
  if (!k_token_major || !k_cache || !aligned16(k_token_major) || !aligned16(k_cache))
    return PA_ERR_INVALID_ARG;
  if (num_blocks < 1 || num_kv_heads < 1) return PA_ERR_INVALID_ARG;
  if (kv_dtype != PA_KV_F16 && kv_dtype != PA_KV_E4M3) return PA_ERR_INVALID_ARG;
  const int64_t slice = (int64_t)PA_BLOCK_SIZE * PA_HEAD_DIM * (kv_dtype == PA_KV_E4M3 ? 1 : 2);
  if (num_blocks > INT64_MAX / 4 / slice / num_kv_heads) return PA_ERR_UNSUPPORTED;
  const int64_t slices = num_blocks * num_kv_heads;
  const uintptr_t a = reinterpret_cast<uintptr_t>(k_token_major);
  const uintptr_t b = reinterpret_cast<uintptr_t>(k_cache);
  const uintptr_t n = (uintptr_t)(slices * slice);
  if (a < b + n && b < a + n) return PA_ERR_INVALID_ARG;  // the two must not overlap
  if (pa::launch_pack_k(k_token_major, k_cache, slices, kv_dtype == PA_KV_E4M3,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

// Streaming-read grid: one 256-thread work-group per CU, i.e. 4 waves per
// CU each with 8 KiB of loads in flight, the 32 KiB per CU the decode's
// streaming shape also holds.  Measured on MI355X: 7.17-7.23 TB/s over
// 1 GiB and 4 GiB, against 6.80-7.02 TB/s for 2..32 work-groups per CU
// (more loads in flight only queue).
int stream_groups() { return (int)current_device_info().cus; }

size_t paged_attn_stream_read_sink_bytes(size_t bytes) {
  (void)bytes;
  return 16 * (size_t)stream_groups();
}

int paged_attn_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || (bytes & 15u) || !aligned16(buf) || !aligned16(sink))
    return PA_ERR_INVALID_ARG;
  if (pa::launch_stream_read(buf, bytes, sink, stream_groups(),
                             static_cast<hipStream_t>(stream)) != hipSuccess)
    return PA_ERR_HIP;
  return PA_OK;
}

const char* paged_attn_error_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or option";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int paged_attn_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
