// Paged decode attention kernels for gfx950 (CDNA4, wave64).
//
// Method (asynchronous-KV-prefetch review, sections 3.2-3.4 and 4.1): a
// work-group owns the block range [s, e) of one (sequence, KV head); its W
// wavefronts walk the range with stride W (wave i takes s+i, s+i+W, ...; the
// KV-cache-prefetching article, section 2.2, gives the same assignment for a
// 4-warp block).  Before computing block j a wavefront issues the fetch of
// block j+W, so the memory latency of the next block overlaps the compute of
// the current one.  Q*K^T is computed per block against the Q heads held in
// registers, then logits times V.
//
// Lane layout for one 16-token x 128-dim fp16 block (4 KiB, contiguous):
//   lane l = 16 r + c  (row r = 0..3, column c = 0..15)
//   load i (0..3) reads token 4i + r, dims 8c..8c+7: 16 bytes at byte offset
//   1024 i + 16 l, so every load instruction covers 1 KiB of whole 128 B lines.
// Q.K: each lane does 4 v_dot2_f32_f16 over its 8 dims; a 16-lane DPP
// butterfly leaves the token's full dot product in every lane of the row.
// Each row keeps its own online-softmax state (m, l, acc[8 dims per lane])
// over the tokens 4i + r it owns, so the hot loop needs no cross-row traffic.
// The 4 rows and then the W waves are merged once at the end.
//
// Look-ahead modes (PF): 0 none; 1 an L2 / Infinity-Cache touch of every
// 128 B line of block j+W (one dword per lane, value discarded); 2 block j+W
// loaded into a second register buffer before block j is computed; 3 both,
// with the touch moved to block j+2W.  The arithmetic is the same code in
// every mode, so results are bitwise identical.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kT = 16;
constexpr int kWave = 64;
constexpr int kBlockHeadBytes = kD * kT * 2;  // 4096

// DPP controls (gfx9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same bits
// (each step adds two operands that are the same pair on both partners).
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half2_t as_h2(uint32_t u) {
  return __builtin_bit_cast(half2_t, u);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

struct BlockBuf {
  u32x4 k[4];
  u32x4 v[4];
};

// ---------------------------------------------------------------------------
template <int G, int PF, bool DBG>
__global__ void __launch_bounds__(G <= 8 ? 512 : 256)
pa_decode_kernel(const DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  int32_t* bt_s = reinterpret_cast<int32_t*>(smem_raw);
  float* merge_s = reinterpret_cast<float*>(smem_raw + a.lds_bt_bytes);

  const int p = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int W = blockDim.x / kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int r = lane >> 4;
  const int c = lane & 15;

  int ctx = a.ctx[b];
  const int tab_tokens = a.MB * kT;
  if (ctx > tab_tokens) {
    if (DBG && tid == 0 && a.dbg_err) atomicOr(a.dbg_err, 2);
    ctx = tab_tokens;
  }
  const int nb = ctx > 0 ? (ctx + kT - 1) / kT : 0;
  const int s = p * a.PB;
  const int e = min(nb, s + a.PB);

  if (s >= e) {
    // Nothing to attend in this partition.  With one partition the output
    // row is written here (context <= 0 gives zeros); otherwise the reduce
    // kernel only reads partitions that hold blocks.
    if (a.P == 1) {
      for (int idx = tid; idx < G * kD; idx += blockDim.x) {
        const int h = idx / kD, d = idx % kD;
        a.out[((int64_t)b * a.Hq + kvh * G + h) * kD + d] = 0;
      }
    }
    return;
  }

  // Stage this partition's block-table slice in LDS.
  const int32_t* bt_row = a.bt + (int64_t)b * a.MB;
  for (int i = tid; i < e - s; i += blockDim.x) bt_s[i] = bt_row[s + i];

  // Q heads of this KV head: 8 dims (16 B) per lane per head.
  half2_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(
        a.q + ((int64_t)b * a.Hq + kvh * G + h) * kD + 8 * c);
    qv[h][0] = as_h2(w4.x);
    qv[h][1] = as_h2(w4.y);
    qv[h][2] = as_h2(w4.z);
    qv[h][3] = as_h2(w4.w);
  }
  __syncthreads();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
  }

  const unsigned char* kbase =
      reinterpret_cast<const unsigned char*>(a.k) + (int64_t)kvh * kBlockHeadBytes;
  const unsigned char* vbase =
      reinterpret_cast<const unsigned char*>(a.v) + (int64_t)kvh * kBlockHeadBytes;
  const int lane_off = lane * 16;

  auto load_block = [&](BlockBuf& buf, int64_t ph) {
    const unsigned char* kb = kbase + ph * a.blk_bytes + lane_off;
    const unsigned char* vb = vbase + ph * a.blk_bytes + lane_off;
#pragma unroll
    for (int i = 0; i < 4; ++i) buf.k[i] = *reinterpret_cast<const u32x4*>(kb + 1024 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) buf.v[i] = *reinterpret_cast<const u32x4*>(vb + 1024 * i);
  };

  // One dword per lane: lanes 0-31 cover the 32 lines of the K block, lanes
  // 32-63 those of the V block.
  auto touch_block = [&](int64_t ph) -> uint32_t {
    const unsigned char* base = (lane < 32 ? kbase : vbase) + ph * a.blk_bytes;
    return *reinterpret_cast<const uint32_t*>(base + (lane & 31) * 128);
  };

  auto trace_put = [&](int j, int slot, int value) {
    if (DBG && a.dbg_trace && lane == 0)
      a.dbg_trace[(((int64_t)b * a.Hkv + kvh) * a.MB + j) * 2 + slot] = value;
  };

  auto compute = [&](BlockBuf& buf, int j) {
    if (DBG && a.dbg_k) {
      unsigned char* dst = reinterpret_cast<unsigned char*>(a.dbg_k) +
                           ((((int64_t)b * a.Hkv + kvh) * a.MB + j) * kT) * kD * 2 +
                           lane_off;
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(dst + 1024 * i) = buf.k[i];
    }
    const int tok0 = j * kT + r;  // this row's token for i = 0; +4 per i
    const bool tail = j * kT + kT > ctx;
    if (tail) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (tok0 + 4 * i >= ctx) buf.v[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float sc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float d = 0.f;
        d = __builtin_amdgcn_fdot2(qv[h][0], as_h2(buf.k[i].x), d, false);
        d = __builtin_amdgcn_fdot2(qv[h][1], as_h2(buf.k[i].y), d, false);
        d = __builtin_amdgcn_fdot2(qv[h][2], as_h2(buf.k[i].z), d, false);
        d = __builtin_amdgcn_fdot2(qv[h][3], as_h2(buf.k[i].w), d, false);
        sc[i] = row_sum16(d) * a.scale_log2;
      }
      float m_use;
      float m_new;
      if (tail) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 4 * i >= ctx) sc[i] = -INFINITY;
        m_new = fmaxf(m[h], fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        m_use = m_new == -INFINITY ? 0.f : m_new;
      } else {
        m_new = fmaxf(m[h], fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        m_use = m_new;
      }
      const float alpha = fast_exp2(m[h] - m_use);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - m_use);
      l[h] = l[h] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m[h] = m_new;
#pragma unroll
      for (int d = 0; d < 8; ++d) acc[h][d] *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t vw[4] = {buf.v[i].x, buf.v[i].y, buf.v[i].z, buf.v[i].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const half2_t hv = as_h2(vw[u]);
          acc[h][2 * u] = __builtin_fmaf(pr[i], (float)hv.x, acc[h][2 * u]);
          acc[h][2 * u + 1] = __builtin_fmaf(pr[i], (float)hv.y, acc[h][2 * u + 1]);
        }
      }
    }
  };

  // ---- the block walk -----------------------------------------------------
  // Wave `wave` runs n_it iterations; iteration it computes block j0 + it*W,
  // whose table entry is bt_s[wave + it*W].  The entries of iterations
  // [base, base+64) and [base+64, base+128) are held one per lane in btv0 /
  // btv1 and read with v_readlane, so no block address waits on memory; the
  // pair moves on by 64 when the walk crosses a chunk.
  const int j0 = s + wave;
  const int n_it = j0 < e ? (e - j0 + W - 1) / W : 0;
  const int nslice = e - s;
  auto bt_chunk = [&](int base) -> int {
    const int idx = wave + W * (base + lane);
    return idx < nslice ? bt_s[idx] : 0;
  };
  int chunk_base = 0;
  int btv0 = bt_chunk(0);
  int btv1 = bt_chunk(64);
  auto phys_it = [&](int it) -> int64_t {
    const int v0 = __builtin_amdgcn_readlane(btv0, it & 63);
    const int v1 = __builtin_amdgcn_readlane(btv1, it & 63);
    int ph = it - chunk_base < 64 ? v0 : v1;
    if (DBG) {
      if (ph < 0 || (int64_t)ph >= a.NB) {
        if (lane == 0 && a.dbg_err) atomicOr(a.dbg_err, 1);
        ph = 0;
      }
    }
    return (int64_t)ph;
  };
  auto advance = [&](int it) {
    if (((it + 1) & 63) == 0) {
      chunk_base += 64;
      btv0 = btv1;
      btv1 = bt_chunk(chunk_base + 64);
    }
  };
  uint32_t sink = 0;

  // The steady-state loops issue their look-ahead loads unconditionally (the
  // last iterations are peeled), so the compiler's wait before block j's
  // first use counts block j+W's loads as still in flight.
  if constexpr (PF <= 1) {
    uint32_t pend = 0;
    int it = 0;
    for (; it + 1 < n_it; ++it) {  // block j+W exists
      const int j = j0 + it * W;
      BlockBuf buf;
      load_block(buf, phys_it(it));
      uint32_t got = 0;
      if (PF == 1) {
        got = touch_block(phys_it(it + 1));
        trace_put(j + W, 1, wave);
      }
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j);
      if (PF == 1) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
    }
    if (it < n_it) {  // this wave's last block: nothing left to fetch ahead
      const int j = j0 + it * W;
      BlockBuf buf;
      load_block(buf, phys_it(it));
      trace_put(j, 0, (wave << 16) | it);
      compute(buf, j);
    }
    sink ^= pend;
  } else {
    BlockBuf bufA, bufB;
    uint32_t pend = 0;
    auto step = [&](BlockBuf& cur, BlockBuf& nxt, int it) {
      const int j = j0 + it * W;
      load_block(nxt, phys_it(it + 1));
      trace_put(j + W, 1, wave);
      uint32_t got = 0;
      if (PF == 3) got = touch_block(phys_it(it + 2));
      trace_put(j, 0, (wave << 16) | it);
      compute(cur, j);
      if (PF == 3) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
    };
    int it = 0;
    if (n_it > 0) load_block(bufA, phys_it(0));
    for (; it + 3 < n_it; it += 2) {  // blocks it+1 .. it+3 exist
      step(bufA, bufB, it);
      step(bufB, bufA, it + 1);
    }
    for (; it < n_it; ++it) {  // at most 3 left; bufA holds block `it`
      const int j = j0 + it * W;
      if (it + 1 < n_it) {
        load_block(bufB, phys_it(it + 1));
        trace_put(j + W, 1, wave);
      }
      uint32_t got = 0;
      if (PF == 3 && it + 2 < n_it) got = touch_block(phys_it(it + 2));
      trace_put(j, 0, (wave << 16) | it);
      compute(bufA, j);
      if (PF == 3) {
        sink ^= pend;
        pend = got;
      }
      advance(it);
      bufA = bufB;
    }
    sink ^= pend;
  }
  // The touched data is discarded; this keeps the loads alive without ever
  // storing (a.sink_enable is 0 in every call).
  if (a.sink_enable && sink == 0x9E3779B9u && lane == 0) a.sink[0] = (int32_t)sink;

  // ---- merge the 4 rows of each wave (lanes l, l^16, l^32, l^48) ----------
#pragma unroll
  for (int step = 16; step <= 32; step *= 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], step);
      const float lo = __shfl_xor(l[h], step);
      const float M = fmaxf(m[h], mo);
      const float Mu = M == -INFINITY ? 0.f : M;
      const float as = fast_exp2(m[h] - Mu);
      const float ao = fast_exp2(mo - Mu);
      l[h] = l[h] * as + lo * ao;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float oo = __shfl_xor(acc[h][d], step);
        acc[h][d] = acc[h][d] * as + oo * ao;
      }
      m[h] = M;
    }
  }

  // ---- merge the W waves through LDS --------------------------------------
  constexpr int kRec = kD + 2;  // m, l, o[128]
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* rec = merge_s + (wave * G + h) * kRec;
      if (c == 0) {
        rec[0] = m[h];
        rec[1] = l[h];
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) rec[2 + 8 * c + d] = acc[h][d];
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * kD; idx += blockDim.x) {
    const int h = idx / kD, d = idx % kD;
    float M = -INFINITY;
    for (int w = 0; w < W; ++w) M = fmaxf(M, merge_s[(w * G + h) * kRec]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, O = 0.f;
    for (int w = 0; w < W; ++w) {
      const float* rec = merge_s + (w * G + h) * kRec;
      const float al = fast_exp2(rec[0] - Mu);
      L += al * rec[1];
      O += al * rec[2 + d];
    }
    const int64_t row = (int64_t)b * a.Hq + kvh * G + h;
    if (a.P == 1) {
      a.out[row * kD + d] = f32_to_f16_bits(O / L);
    } else {
      const int64_t pr = row * a.P + p;
      if (d == 0) {
        a.ws_ml[pr * 2] = M;
        a.ws_ml[pr * 2 + 1] = L;
      }
      a.ws_o[pr * kD + d] = O;
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-partition combine: one work-group of 128 threads per (sequence, head).
__global__ void __launch_bounds__(128) pa_reduce_kernel(const DecodeArgs a) {
  const int row = blockIdx.x;  // b * Hq + h
  const int b = row / a.Hq;
  const int d = threadIdx.x;
  int ctx = a.ctx[b];
  ctx = min(ctx, a.MB * kT);
  const int nb = ctx > 0 ? (ctx + kT - 1) / kT : 0;
  const int np = (nb + a.PB - 1) / a.PB;
  if (np == 0) {
    a.out[(int64_t)row * kD + d] = 0;
    return;
  }
  const float* ml = a.ws_ml + (int64_t)row * a.P * 2;
  const float* o = a.ws_o + (int64_t)row * a.P * kD;
  float M = -INFINITY;
  for (int q = 0; q < np; ++q) M = fmaxf(M, ml[2 * q]);
  float L = 0.f, O = 0.f;
  for (int q = 0; q < np; ++q) {
    const float al = fast_exp2(ml[2 * q] - M);
    L += al * ml[2 * q + 1];
    O += al * o[(int64_t)q * kD + d];
  }
  a.out[(int64_t)row * kD + d] = f32_to_f16_bits(O / L);
}

// ---------------------------------------------------------------------------
// Streaming-read ceiling: every 16-byte word of buf read once.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ buf,
                                                          int64_t n16, u32x4* sink) {
  const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  u32x4 x = {0u, 0u, 0u, 0u};
  for (; i + 3 * nthreads < n16; i += 4 * nthreads) {
    const u32x4 a0 = buf[i];
    const u32x4 a1 = buf[i + nthreads];
    const u32x4 a2 = buf[i + 2 * nthreads];
    const u32x4 a3 = buf[i + 3 * nthreads];
    x ^= a0 ^ a1 ^ a2 ^ a3;
  }
  for (; i < n16; i += nthreads) x ^= buf[i];
  // reduce within the work-group so only one value per group is stored
  __shared__ u32x4 red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] ^= red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// ---------------------------------------------------------------------------
// Launchers.

template <int G, int PF, bool DBG>
static hipError_t launch_decode_t(const DecodeArgs& a, dim3 grid, dim3 block,
                                  size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((pa_decode_kernel<G, PF, DBG>), grid, block, lds, st, a);
  return hipGetLastError();
}

typedef hipError_t (*decode_fn)(const DecodeArgs&, dim3, dim3, size_t, hipStream_t);

template <int G>
static decode_fn pick_pf(int pf, bool dbg) {
  switch (pf * 2 + (dbg ? 1 : 0)) {
    case 0: return launch_decode_t<G, 0, false>;
    case 1: return launch_decode_t<G, 0, true>;
    case 2: return launch_decode_t<G, 1, false>;
    case 3: return launch_decode_t<G, 1, true>;
    case 4: return launch_decode_t<G, 2, false>;
    case 5: return launch_decode_t<G, 2, true>;
    case 6: return launch_decode_t<G, 3, false>;
    case 7: return launch_decode_t<G, 3, true>;
  }
  return nullptr;
}

static decode_fn pick(int g, int pf, bool dbg) {
  switch (g) {
    case 1: return pick_pf<1>(pf, dbg);
    case 2: return pick_pf<2>(pf, dbg);
    case 3: return pick_pf<3>(pf, dbg);
    case 4: return pick_pf<4>(pf, dbg);
    case 5: return pick_pf<5>(pf, dbg);
    case 6: return pick_pf<6>(pf, dbg);
    case 7: return pick_pf<7>(pf, dbg);
    case 8: return pick_pf<8>(pf, dbg);
    case 9: return pick_pf<9>(pf, dbg);
    case 10: return pick_pf<10>(pf, dbg);
    case 11: return pick_pf<11>(pf, dbg);
    case 12: return pick_pf<12>(pf, dbg);
    case 13: return pick_pf<13>(pf, dbg);
    case 14: return pick_pf<14>(pf, dbg);
    case 15: return pick_pf<15>(pf, dbg);
    case 16: return pick_pf<16>(pf, dbg);
  }
  return nullptr;
}

hipError_t launch_decode(const DecodeArgs& a, int g, int pf, bool dbg, int waves,
                         hipStream_t st) {
  decode_fn fn = pick(g, pf, dbg);
  if (!fn) return hipErrorInvalidValue;
  const dim3 grid(a.P, a.Hkv, a.B);
  const dim3 block(kWave * waves);
  return fn(a, grid, block, decode_lds_bytes(a.PB, g, waves), st);
}

hipError_t launch_reduce(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(pa_reduce_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(kD), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, void* sink, int groups,
                              hipStream_t st) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(groups), dim3(256), 0, st,
                     reinterpret_cast<const u32x4*>(buf), (int64_t)(bytes / 16),
                     reinterpret_cast<u32x4*>(sink));
  return hipGetLastError();
}

}  // namespace pa
