// Internal interface between the C ABI (pa_api.cpp) and the kernels
// (pa_kernels.hip).  Not installed; the public interface is paged_attn.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Everything a decode launch needs, passed by value as the kernel argument.
struct DecodeArgs {
  const uint16_t* q;     // [B][Hq][128] fp16
  const void* k;         // fp16 [NB][Hkv][16 dim groups][16 tokens][8], or
                         // E4M3 [NB][Hkv][8 dim groups][16 tokens][16]
  const void* v;         // fp16 or E4M3 [NB][Hkv][16 tokens][128]
  const int32_t* bt;     // [B][MB]
  const int32_t* ctx;    // [B]
  uint16_t* out;         // [B][Hq][128] fp16
  float* ws_ml;          // [B][Hq][P][2]   (max in log2 units, sum)
  float* ws_o;           // [B][Hq][P][128] unnormalised output (the workspace's start)
  uint16_t* dbg_k;       // see pa_options.debug_gather_k
  int32_t* dbg_trace;    // see pa_options.debug_trace
  int32_t* dbg_err;      // see pa_options.debug_error_word
  int64_t* dbg_timeline; // see pa_options.debug_timeline
  int32_t* sink;         // never written while sink_enable == 0
  float scale_log2;      // scale * log2(e) (times the K scale for E4M3 caches)
  float v_scale;         // 1, or the V scale of an E4M3 cache
  int B, Hq, Hkv, MB;
  int G;                 // query heads per KV head, 1..16
  int P;                 // partitions in the grid
  int PB;                // blocks per partition
  int64_t NB;            // pool blocks
  int64_t k_blk, v_blk;    // bytes from one physical block to the next, K and V
  int64_t k_head, v_head;  // bytes from one KV head's slice to the next
  int lds_bt_bytes;      // LDS bytes reserved for the block-table slice
  int pf_dist;           // L2-touch distance in iterations of a wave, 1..63
  int sink_enable;
  int rank_seqs;         // 1: grid row r takes the sequence of rank r (most blocks first)
  // Balanced split (balanced = 1): grid (Hkv, nslot); the partition size is
  // chosen on the device from the context lengths, a multiple of the wave
  // count between PB and pb_max, so that all sequences need at most nslot
  // partitions.  P is then the workspace's partition stride (the most
  // partitions one sequence can get) and ws_np[b] receives sequence b's
  // partition count for the reduce.
  int balanced;
  int nslot;
  int pb_max;
  int k_uniform;         // min(nslot / B, P): partitions per sequence of a uniform batch
  int chain;             // 2: grid row y walks sequence ranks y and B-1-y in turn (P == 1)
  // Even split (even = 1): grid (S); share c takes blocks [c T / S, (c + 1)
  // T / S) of the T (block, KV head) pairs of all sequences, KV-head-major
  // (head 0's sequences in order, then head 1's, ...).  A piece of a unit
  // that crosses a share boundary goes to record 2c (the share's first
  // piece) or 2c + 1 (its last) of ws_o / ws_ml, [2 S][G] rows, and the
  // share holding a unit's block 0 writes ws_np[2 u] = its record and
  // ws_np[2 u + 1] = the unit's piece count (u = b Hkv + kvh).  Piece j > 0
  // of a unit is record 2 (c0 + j); a share with no blocks leaves an empty
  // record (m = -inf, l = 0, o = 0) at 2c.
  int even;
  int shares;            // S, the even split's grid
  int even_kappa;        // blocks a piece change is charged in the share sizes
  int32_t* ws_np;
};

// floats of the even split's records: 2 per share, g rows of 128 + 2
inline size_t even_records(int64_t shares, int g) {
  return (size_t)2 * shares * g * (128 + 2);
}

// Partials the reduce kernel merges with one memory round trip, and the
// partition size from which the auto plans let a sequence have more of them
// (more, smaller partitions cost the reduce more than the extra CUs bring).
constexpr int kReduceRegs = 8;
constexpr int kReduceBigPartition = 64;

inline int lds_bt_bytes_for(int PB) { return ((PB * 4) + 15) / 16 * 16; }

// LDS of the sequence ranking: B block counts padded to a multiple of 4,
// then the selected sequence.  It overlays the block-table slice and the
// merge area, which are written only after the ranking is done.
inline size_t rank_lds_bytes(int B) { return (size_t)((B + 3) / 4 * 4) * 4 + 16; }

// LDS the compiler adds beside a kernel's dynamic allocation, at most (the
// decode kernel's is 256 B: the scratch word of __syncthreads_or).  Plans
// keep dynamic + this within the device's LDS per work-group.
constexpr size_t kCompilerLdsBytes = 1024;

// Dynamic LDS that holds at most `cap` work-groups on a CU with `per_cu`
// bytes: per_cu / cap rounded down to 1 KiB, less kCompilerLdsBytes (so
// that cap of them fit with their compiler LDS whatever the allocation
// granularity up to 1 KiB, and cap + 1 do not).
inline size_t residency_lds_bytes(size_t per_cu, int cap) {
  const size_t share = per_cu / (size_t)cap / 1024 * 1024;
  return share > kCompilerLdsBytes ? share - kCompilerLdsBytes : 0;
}

// `slots`: the LDS-staged look-ahead's per-wave slots, which overlay the
// merge records (they are free by the time the records are written).
inline size_t decode_lds_bytes(int PB, int g, int waves, int B, bool rank, size_t slots = 0) {
  const size_t rec = (size_t)waves * g * (128 + 2) * 4;
  const size_t main = (size_t)lds_bt_bytes_for(PB) + (rec > slots ? rec : slots);
  const size_t r = rank ? rank_lds_bytes(B) : 0;
  return main > r ? main : r;
}

// The two-loop walk adds the range's scores (PB*16*g fp32) and one maximum
// per wave and head after the merge records.
inline size_t two_loop_lds_bytes(int PB, int g, int waves, int B, bool rank) {
  const size_t main = decode_lds_bytes(PB, g, waves, B, false) + (size_t)PB * 16 * g * 4 +
                      (size_t)waves * g * 4;
  const size_t r = rank ? rank_lds_bytes(B) : 0;
  return main > r ? main : r;
}

// Bytes of the per-device scratch array of paged_attn_decode_noalloc
// (PA_NOALLOC_SCRATCH_BYTES in paged_attn.h).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
// The current device's address of that array (looked up on the first call
// on each device, then cached).
hipError_t noalloc_scratch(void** ptr);

hipError_t launch_decode_two_loop(const DecodeArgs& a, int pf, int waves, size_t lds,
                                  hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int pf, bool dbg, bool kv8, int waves,
                         size_t lds, hipStream_t st);
hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st);
hipError_t launch_pack_k(const void* in, void* out, int64_t slices, bool kv8, hipStream_t st);
hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int groups,
                              hipStream_t st);

}  // namespace pa
