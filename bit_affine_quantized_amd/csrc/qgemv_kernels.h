// qgemv_kernels.h — device code of the row product (templates), shared by
// the per-width translation units and the host code.
#pragma once
// Row product kernels for gfx950 (MI355X).
//
// y[i,n] = epi( sum_g ( s[n,g] * A[i,n,g] + b[n,g] * X[i,g] ) )
//   A[i,n,g] = sum over the 32-code units of group g of (fp32 chain of
//              exact bf16 code x bf16 activation products),
//   X[i,g]   = sum of the activations over the same units.
// The affine form and the fp32 group sums follow "Qwen3.8-Flash-Next faster
// kernels in Zig engine - #788" (commit "...row kernel at every MLX width":
// an fp64 product from the MLX reference dequantization is the check;
// commit "2-bit prompt product": codes enter exactly, with no offset) and
// "Qwen3.8-Flash-Next support for oQ in Zig engine - #774" ("Exactness",
// "Precision": activations stay bf16, group sums fp32).
//
// Design for CDNA4 (what differs from the pages' Metal lane kernels):
//  * One output column (a weight row) is shared by LPR lanes of a 64-wide
//    wave; each lane owns whole 128-bit-aligned chunks of the row's
//    bitstream (16/48/16/80/48/32 bytes for 2/3/4/5/6/8 bits), so every
//    code fetch is a global_load_dwordx4 and no code straddles two lanes.
//  * Codes are cut once (v_bfe/v_alignbit or byte converts, specialised per
//    width at compile time), converted to exact bf16 pairs and multiplied by
//    bf16 activation pairs with v_dot2c_f32_bf16 (fp32 accumulate): one
//    instruction per two products, and activations never leave bf16.
//  * The activation window is staged once per block in LDS, laid out so the
//    lanes' 16-byte reads are conflict-free; per-unit activation sums are
//    computed there once.
//  * Lanes reduce with a fixed xor butterfly; no float atomics anywhere.
//
// Row invariance (a row's bits are the same alone, in any window, and in
// plain, strided and indexed calls — commit "...row kernel at every MLX
// width"): the lane->K mapping, the unit order, the dot2 chain, the group
// epilogue and the butterfly depend on (bits, group, N, K) only.  The
// window size changes how many rows run side by side, never the operations
// any one row sees.  Built with -ffp-contract=off; every fused op is an
// explicit builtin.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <new>

#include "qgemv.h"

namespace qg {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSlots = 64;
constexpr int kMaxList = QGEMV_MAX_WINDOW * kMaxSlots;
constexpr int kMaxSeg = 4;    // members per run of a fused stack
constexpr int kMaxRuns = 8;   // runs per fused stack
// 160 KiB of LDS per CU on gfx950, less the kernels' static arrays.
constexpr size_t kMaxDynamicLds = 160 * 1024 - 8 * 1024;
constexpr size_t kMaxMfmaLds = 160 * 1024 - 1024;   // the MFMA kernels' static LDS is a few hundred bytes

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Output columns each lane carries side by side (more loads in flight,
// activations read from LDS once for all of them).
template <int B, int MB> struct RowsPerLane {
  static constexpr int v = (MB == 1) ? ((B == 2 || B == 4 || B == 8) ? 4 : 2) : (MB >= 8 ? 1 : 2);
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Two fp32 integers (< 2^8, so their low 16 bits are zero) -> bf16 pair
// {lo = f0, hi = f1}, exactly.
__device__ __forceinline__ uint32_t pack_bf16x2(float f0, float f1) {
  return __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Code J of a 32-code unit held in B words (bit J*B of the unit's stream).
template <int B, int J>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w) {
  constexpr int o = J * B, wi = o / 32, sh = o % 32;
  if constexpr (sh + B <= 32) {
    return __builtin_amdgcn_ubfe(w[wi], sh, B);
  } else {
    return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
  }
}

// Byte pair {c0, c1} (codes 0..15) -> exact bf16 pair, two codes per
// instruction: a byte holding c < 16 reads as an fp8 e4m3 value c * 2^-9
// (exponent field 0 or 1, both on the same linear scale), and the scaled
// conversion multiplies by 2^9 exactly.  hi selects bytes 2,3 instead of 0,1.
template <bool HI>
__device__ __forceinline__ uint32_t bytes_to_bf16x2(uint32_t bytes) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bytes, 512.0f, HI));
}

template <int B, int P, int NPAIR = 16>
__device__ __forceinline__ void unpack_pairs_odd(const uint32_t* w, uint32_t* q) {
  if constexpr (P < NPAIR) {
    if constexpr (B == 3) {
      // two 3-bit codes -> bytes {c0, c1} -> one conversion
      q[P] = bytes_to_bf16x2<false>(unit_code<B, 2 * P>(w) | (unit_code<B, 2 * P + 1>(w) << 8));
    } else {
      q[P] = pack_bf16x2(static_cast<float>(unit_code<B, 2 * P>(w)),
                         static_cast<float>(unit_code<B, 2 * P + 1>(w)));
    }
    unpack_pairs_odd<B, P + 1, NPAIR>(w, q);
  }
}

// NC codes (NC*B a multiple of 32) held in NC*B/32 words -> NC/2 exact bf16
// pairs q[p] = {code slot_code<B>(2p), code slot_code<B>(2p+1)}.  2- and
// 4-bit codes are split into bytes with masks and converted two per
// instruction, which pairs them in the order slot_code gives; the
// activations are staged in the same order, so each pair still meets its
// own two activations.
template <int B>
__host__ __device__ constexpr int slot_code(int slot) {
  if constexpr (B == 2) {
    // per 16-code word: t_s = (w >> 2s) & 0x03030303 holds codes s, 4+s, 8+s, 12+s
    const int wi = slot / 16, r = slot % 16, sft = r / 4, half = (r / 2) % 2, el = r % 2;
    return 16 * wi + sft + 4 * el + 8 * half;
  } else if constexpr (B == 4) {
    // per 8-code word: low nibbles hold codes 0,2,4,6; high nibbles 1,3,5,7
    const int wi = slot / 8, r = slot % 8, b = r / 2, el = r % 2;
    return 8 * wi + b / 2 + 4 * (b % 2) + 2 * el;
  } else {
    return slot;
  }
}

template <int B, int NC>
__device__ __forceinline__ void unpack_codes(const uint32_t* w, uint32_t* q) {
  static_assert((NC * B) % 32 == 0 && NC % 16 == 0, "whole words");
  if constexpr (B == 8) {
#pragma unroll
    for (int wi = 0; wi < NC / 4; ++wi) {
      const uint32_t v = w[wi];
      q[2 * wi] = pack_bf16x2(static_cast<float>(v & 0xffu), static_cast<float>((v >> 8) & 0xffu));
      q[2 * wi + 1] = pack_bf16x2(static_cast<float>((v >> 16) & 0xffu), static_cast<float>(v >> 24));
    }
  } else if constexpr (B == 4) {
#pragma unroll
    for (int wi = 0; wi < NC / 8; ++wi) {
      const uint32_t lo = w[wi] & 0x0f0f0f0fu;
      const uint32_t hi = (w[wi] >> 4) & 0x0f0f0f0fu;
      q[4 * wi] = bytes_to_bf16x2<false>(lo);
      q[4 * wi + 1] = bytes_to_bf16x2<true>(lo);
      q[4 * wi + 2] = bytes_to_bf16x2<false>(hi);
      q[4 * wi + 3] = bytes_to_bf16x2<true>(hi);
    }
  } else if constexpr (B == 2) {
#pragma unroll
    for (int wi = 0; wi < NC / 16; ++wi) {
#pragma unroll
      for (int sft = 0; sft < 4; ++sft) {
        const uint32_t t = (w[wi] >> (2 * sft)) & 0x03030303u;
        q[8 * wi + 2 * sft] = bytes_to_bf16x2<false>(t);
        q[8 * wi + 2 * sft + 1] = bytes_to_bf16x2<true>(t);
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < NC / 32; ++u) unpack_pairs_odd<B, 0>(w + u * B, q + 16 * u);
    // a half unit (16 codes in whole words: 6 bits)
    if constexpr (NC % 32 == 16) unpack_pairs_odd<B, 0, 8>(w + (NC / 32) * B, q + 16 * (NC / 32));
  }
}

// Activation pair p of an NC-code unit in the order unpack_codes pairs the
// codes: x holds the unit's activations as natural bf16 pairs.
template <int B>
__device__ __forceinline__ uint32_t slot_pair(const uint32_t* x, int p) {
  const int a = slot_code<B>(2 * p), b = slot_code<B>(2 * p + 1);
  const uint32_t sel = ((a & 1) ? 0x0302u : 0x0100u) | ((b & 1) ? 0x07060000u : 0x05040000u);
  return __builtin_amdgcn_perm(x[b >> 1], x[a >> 1], sel);
}

// WPC words of one lane chunk, as 128-bit loads when the chunk is a whole
// number of 16-byte pieces (always, for the main geometry), else dwords.
template <int WPC>
__device__ __forceinline__ void load_chunk(const uint32_t* __restrict__ p, uint32_t* out) {
  if constexpr (WPC % 4 == 0) {
    const u32x4* p4 = reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < WPC / 4; ++i) {
      const u32x4 v = __builtin_nontemporal_load(p4 + i);
      out[4 * i] = v.x;
      out[4 * i + 1] = v.y;
      out[4 * i + 2] = v.z;
      out[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < WPC; ++i) out[i] = __builtin_nontemporal_load(p + i);
  }
}

struct Params {
  // What a block needs before its first loads comes first, in the first 104
  // bytes of the argument segment, so that the kernels read it in one round
  // of scalar loads.
  const uint32_t* w;        // [E][N][WPR]
  const uint16_t* scales;   // [E][N][GPR]
  const uint16_t* biases;
  const uint16_t* x;        // [M][K] bf16
  int64_t n;                // output columns
  int64_t k;
  int64_t wpr;              // words per row
  int64_t gpr;              // groups per row
  int32_t m;                // window rows
  int32_t tiles;            // column tiles per expert
  int32_t ks_shift;         // matrix-core form: log2(ksplit)
  int32_t gpp;              // matrix-core form: load groups per K-part
  float inv_units;          // matrix-core form: 1 / (k / 32), rounded (see split_units)
  int32_t slots;            // indexed only
  const int32_t* idx;       // indexed: [M][slots]
  // the rest
  float* y;
  int64_t ldy;              // plain/strided row stride of y
  int32_t n_experts;
  int32_t epi;
  int32_t lpr;              // lanes per output column (power of two <= 64)
  int32_t cpl;              // chunks per lane
  int32_t nchunks;          // chunks per row = lpr * cpl
  int32_t indexed;          // 0: plain/strided, 1: indexed
  int32_t vec_groups;       // scales/biases aligned for packed loads
  int32_t ksplit;           // matrix-core form: K-parts per column (1, 2 or 4)
  // gate/up pair (matrix-core form): y = silu(gate row) * (up row), the up
  // matrix at w2/scales2/biases2 with the gate's shape; set for the gate/up
  // kernels only, which have the pairing compiled in
  int32_t gateup;
  const uint32_t* w2;
  const uint16_t* scales2;
  const uint16_t* biases2;
  int64_t y_bytes;          // extent of y written by this call (fast kernel stores)
  // column map: rows [seg_row0[s], seg_row0[s+1]) are written at column
  // row + seg_delta[s] (one segment {0, 0} for plain, strided and indexed calls)
  int32_t nseg;
  int32_t seg_row0[kMaxSeg];
  int64_t seg_delta[kMaxSeg];
};
static_assert(offsetof(Params, idx) + sizeof(void*) <= 104, "the first-loads block of Params");

// silu(g) = g / (1 + exp(-g)), fp32, with the device library's expf
__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + expf(-g)); }

__device__ __forceinline__ float apply_epi(float v, int epi) {
  if (epi == QGEMV_EPI_RELU2) return v > 0.0f ? v * v : (v != v ? v : 0.0f);
  return v;
}

// Block-wide list of the (row, slot) pairs routed to `expert`, in index
// order.  Returns the count.
template <int NT = kThreads>
__device__ inline int build_route_list(const int32_t* __restrict__ idx, int total, int expert,
                                int* list, int* wave_cnt) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int base_count = 0;
  for (int base = 0; base < total; base += NT) {
    const int t = base + tid;
    const bool hit = t < total && idx[t] == expert;
    const uint64_t mask = __ballot(hit);
    if (lane == 0) wave_cnt[wv] = __popcll(mask);
    __syncthreads();
    int before = base_count;
    for (int i = 0; i < wv; ++i) before += wave_cnt[i];
    if (hit) {
      const uint64_t lower = lane ? (mask & (~0ull >> (64 - lane))) : 0ull;
      list[before + __popcll(lower)] = t;
    }
    int all = 0;
    for (int i = 0; i < NT / kWave; ++i) all += wave_cnt[i];
    __syncthreads();
    base_count += all;
  }
  return base_count;
}

// Sum of v over the lpr lanes of its column group (a power of two <= 64).
// The tree is fixed: within a 16-lane DPP row, rotate by 8, rotate by 4,
// swap pairs of 2, swap neighbours; then across rows, xor 16 and xor 32.
// Every lane of the group ends with the same bits.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  int o = 0;
  switch (ctrl_sel) {
    case 0: o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false); break;  // row_ror:8
    case 1: o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false); break;  // row_ror:4
    case 2: o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false); break;   // quad [2,3,0,1]
    default: o = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false); break;  // quad [1,0,3,2]
  }
  return v + __int_as_float(o);
}

__device__ __forceinline__ float group_sum(float v, int lpr) {
  if (lpr >= 16) {
    v = dpp_add(v, 0);
    v = dpp_add(v, 1);
    v = dpp_add(v, 2);
    v = dpp_add(v, 3);
    if (lpr >= 32) v += __shfl_xor(v, 16);
    if (lpr >= 64) v += __shfl_xor(v, 32);
  } else {
    if (lpr >= 8) v += __shfl_xor(v, 4);
    if (lpr >= 4) v = dpp_add(v, 2);
    if (lpr >= 2) v = dpp_add(v, 3);
  }
  return v;
}

// Scales (or biases) of one lane chunk: GPC consecutive bf16 values, read as
// one 2-, 4- or 8-byte load when the arrays are aligned for it.
template <int GPC>
__device__ __forceinline__ void load_groups(const uint16_t* __restrict__ p, bool vec, uint32_t* out) {
  if constexpr (GPC == 1) {
    out[0] = __builtin_nontemporal_load(p);
  } else if constexpr (GPC == 2) {
    if (vec) {
      out[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else {
      out[0] = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 16);
    }
  } else {
    static_assert(GPC == 4, "groups per chunk");
    if (vec) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      out[0] = v.x;
      out[1] = v.y;
    } else {
      out[0] = static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 16);
      out[1] = static_cast<uint32_t>(p[2]) | (static_cast<uint32_t>(p[3]) << 16);
    }
  }
}

// bf16 value number i of a packed group array (two per 32-bit word).
template <int GPC>
__device__ __forceinline__ float group_value(const uint32_t* g, int i) {
  if constexpr (GPC == 1) {
    return __uint_as_float(g[0] << 16);
  } else {
    const uint32_t w = g[i >> 1];
    return (i & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
}

template <int B, int G, int UPC, int MB>
__global__ __launch_bounds__(kThreads) void qrow_generic(const Params p) {
  constexpr int WPC = B * UPC;                       // words per lane chunk
  constexpr int UPG = G / 32;                        // units per group
  constexpr int GPC = UPC >= UPG ? UPC / UPG : 1;    // groups per lane chunk
  constexpr int SW = GPC >= 2 ? GPC / 2 : 1;         // packed scale words per chunk
  constexpr int R = RowsPerLane<B, MB>::v;

  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_list[kMaxList];
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_xrow[MB];
  __shared__ int64_t s_yoff[MB];

  const int nchunks = p.nchunks;
  const int units = nchunks * UPC;
  // LDS: x pieces [MB][UPC][4][nchunks] of 16 bytes, then unit sums [MB][UPC][nchunks]
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + static_cast<size_t>(MB) * units * 64);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = tid / kWave;
  const int lpr = p.lpr;
  const int slot = lane / lpr;
  const int li = lane % lpr;
  const int slots_per_wave = kWave / lpr;
  const int tile_rows = kWaves * slots_per_wave * R;
  const int cpl = p.cpl;
  const bool vec = p.vec_groups != 0;

  int expert = 0;
  int total = p.m;
  if (p.indexed) {
    expert = blockIdx.y;
    total = build_route_list(p.idx, p.m * p.slots, expert, s_list, s_wave_cnt);
    if (total == 0) return;
  }
  const uint32_t* __restrict__ wbase = p.w + static_cast<int64_t>(expert) * p.n * p.wpr;
  const uint16_t* __restrict__ sbase = p.scales + static_cast<int64_t>(expert) * p.n * p.gpr;
  const uint16_t* __restrict__ bbase = p.biases + static_cast<int64_t>(expert) * p.n * p.gpr;
  const int n = static_cast<int>(p.n);
  const int wpr = static_cast<int>(p.wpr);
  const int gpr = static_cast<int>(p.gpr);
  // this lane's first row in a tile, before the r offset
  const int lane_row = wv * slots_per_wave * R + slot;
  const int my_tiles = blockIdx.x < p.tiles ? (p.tiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int steps = my_tiles * cpl;

  for (int c0 = 0; c0 < total; c0 += MB) {
    const int mcount = min(MB, total - c0);
    // ---- stage the window: x pieces and per-unit activation sums ----
    if (tid < mcount) {
      const int e = c0 + tid;
      if (p.indexed) {
        const int t = s_list[e];
        const int row = t / p.slots, sl = t % p.slots;
        s_xrow[tid] = row;
        s_yoff[tid] = (static_cast<int64_t>(row) * p.slots + sl) * p.n;
      } else {
        s_xrow[tid] = e;
        s_yoff[tid] = static_cast<int64_t>(e) * p.ldy;
      }
    }
    __syncthreads();
    for (int t = tid; t < mcount * units; t += kThreads) {
      const int mi = t / units, u = t % units;
      const int c = u / UPC, ui = u % UPC;
      const u32x4* src = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(s_xrow[mi]) * p.k +
                                                        static_cast<int64_t>(u) * 32);
      uint32_t xin[16];
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        const u32x4 v = src[pc];
        xin[4 * pc] = v.x;
        xin[4 * pc + 1] = v.y;
        xin[4 * pc + 2] = v.z;
        xin[4 * pc + 3] = v.w;
      }
      // pairs in the order the unpack pairs the codes; X over those pairs
      float X = 0.0f;
      const uint32_t ones = 0x3f803f80u;  // bf16 pair {1, 1}
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        u32x4 o;
        o.x = slot_pair<B>(xin, 4 * pc);
        o.y = slot_pair<B>(xin, 4 * pc + 1);
        o.z = slot_pair<B>(xin, 4 * pc + 2);
        o.w = slot_pair<B>(xin, 4 * pc + 3);
        X = dot2(o.x, ones, X);
        X = dot2(o.y, ones, X);
        X = dot2(o.z, ones, X);
        X = dot2(o.w, ones, X);
        xs[((mi * UPC + ui) * 4 + pc) * nchunks + c] = o;
      }
      xsum[(mi * UPC + ui) * nchunks + c] = X;
    }
    __syncthreads();

    // ---- steps: (tile, chunk) pairs of this block, loads one step ahead ----
    struct Stage {
      uint32_t w[R][WPC];
      uint32_t s[R][SW];
      uint32_t b[R][SW];
    };
    auto load_stage = [&](Stage& st, int step) {
      const int i = step / cpl, j = step - (step / cpl) * cpl;
      const int tile = blockIdx.x + i * gridDim.x;
      const int c = li + lpr * j;
      const int g0 = (c * UPC) / UPG;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(tile * tile_rows + lane_row + r * slots_per_wave, n - 1);
        load_chunk<WPC>(wbase + static_cast<int64_t>(row) * wpr + c * WPC, st.w[r]);
        const int64_t go = static_cast<int64_t>(row) * gpr + g0;
        load_groups<GPC>(sbase + go, vec, st.s[r]);
        load_groups<GPC>(bbase + go, vec, st.b[r]);
      }
    };

    float acc[R][MB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) acc[r][mi] = 0.0f;

    auto compute_stage = [&](const Stage& st, int step) {
      const int i = step / cpl, j = step - (step / cpl) * cpl;
      const int c = li + lpr * j;
#pragma unroll
      for (int ui = 0; ui < UPC; ++ui) {
        uint32_t q[R][16];
#pragma unroll
        for (int r = 0; r < R; ++r) unpack_codes<B, 32>(&st.w[r][ui * B], q[r]);
        const int gi = (UPC >= UPG) ? ui / UPG : 0;
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
          if (mi < mcount) {
            uint32_t xv[16];
#pragma unroll
            for (int pc = 0; pc < 4; ++pc) {
              const u32x4 v = xs[((mi * UPC + ui) * 4 + pc) * nchunks + c];
              xv[4 * pc] = v.x;
              xv[4 * pc + 1] = v.y;
              xv[4 * pc + 2] = v.z;
              xv[4 * pc + 3] = v.w;
            }
            const float X = xsum[(mi * UPC + ui) * nchunks + c];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              float a = 0.0f;
#pragma unroll
              for (int pp = 0; pp < 16; ++pp) a = dot2(q[r][pp], xv[pp], a);
              acc[r][mi] = __builtin_fmaf(group_value<GPC>(st.s[r], gi), a, acc[r][mi]);
              acc[r][mi] = __builtin_fmaf(group_value<GPC>(st.b[r], gi), X, acc[r][mi]);
            }
          }
        }
      }
      if (j == cpl - 1) {
        // ---- the tile's columns are complete: reduce over lanes, store ----
        const int tile = blockIdx.x + i * gridDim.x;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = tile * tile_rows + lane_row + r * slots_per_wave;
#pragma unroll
          for (int mi = 0; mi < MB; ++mi) {
            const float v = group_sum(acc[r][mi], lpr);
            acc[r][mi] = 0.0f;
            if (li == 0 && mi < mcount && row < n) p.y[s_yoff[mi] + row] = apply_epi(v, p.epi);
          }
        }
      }
    };

    // The prefetch is unconditional (its step index is clamped; the last
    // one re-reads the current step, a cache hit) so the loop body is
    // straight-line and each compute waits only for its own stage's loads.
    Stage sa, sb;
    if (steps > 0) {
      load_stage(sa, 0);
      int step = 0;
      for (; step + 1 < steps; step += 2) {
        load_stage(sb, step + 1);
        compute_stage(sa, step);
        load_stage(sa, min(step + 2, steps - 1));
        compute_stage(sb, step + 1);
      }
      if (step < steps) compute_stage(sa, step);
    }
    __syncthreads();  // LDS window reused by the next chunk of routed rows
  }
}

// ---------------------------------------------------------------------------
// Fast kernel: whole 128-bit pieces, perfectly coalesced.
//
// A lane chunk is PPC 16-byte pieces of one row's bitstream holding CPC
// codes: one piece (64/32/16 codes) for 2/4/8 bits, three pieces (128/64
// codes) for 3/6 bits, five pieces (128 codes) for 5 bits.  For 2/4/8 bits
// the lanes of a column group read consecutive pieces of the row, so every
// load instruction is fully coalesced.  For 3/5/6 bits a chunk spans
// several pieces; the wave reads its step's rows as consecutive pieces
// (lane l takes piece l, l+64, ...) and hands each lane its chunk through
// a wave-private LDS buffer (STAGE), or, when LDS is short, each lane
// loads its own chunk (!STAGE).  Both modes feed the same registers to the
// same arithmetic, so a row's bits do not depend on the mode.
// ---------------------------------------------------------------------------

template <int B> struct Geo;
template <> struct Geo<2> { static constexpr int PPC = 1, CPC = 64; };
template <> struct Geo<3> { static constexpr int PPC = 3, CPC = 128; };
template <> struct Geo<4> { static constexpr int PPC = 1, CPC = 32; };
template <> struct Geo<5> { static constexpr int PPC = 5, CPC = 128; };
template <> struct Geo<6> { static constexpr int PPC = 3, CPC = 64; };
template <> struct Geo<8> { static constexpr int PPC = 1, CPC = 16; };

// Output columns per lane of the dot form: 4 at one row for the widths of
// one-piece chunks, 2 for 3, 5 and 6 bits (their chunks hold 3 or 5 pieces;
// measured on MI355X, 2 beat 1 and 4 at one row), fewer for wide windows.
template <int B, int MB> struct FastRows {
  static constexpr int v = (MB == 1) ? ((B == 2 || B == 4 || B == 8) ? 4 : 2) : (MB <= 4 ? 2 : 1);
};

// Sum over a column group of LPR = 16, 32 or 64 lanes: rotate 8, rotate 4,
// swap pairs of 2, swap neighbours inside each 16-lane DPP row, then swap
// the 16-lane halves of each 32 (ds_swizzle), then add the two 32-lane
// halves.  Every lane of the group ends with the same bits.
template <int LPR>
__device__ __forceinline__ float gsum(float v) {
  v = dpp_add(v, 0);
  v = dpp_add(v, 1);
  v = dpp_add(v, 2);
  v = dpp_add(v, 3);
  // (the swizzle and readlane builtins move 32-bit integers: bit-cast)
  if constexpr (LPR >= 32) v = v + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  if constexpr (LPR >= 64)
    v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
        __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  return v;
}

// Lanes with nothing to load or store aim at buffer offset kNoOffset, and
// every buffer resource spans at most kNoOffset bytes, so that offset is
// always past the end: such loads read 0 and such stores are dropped.  The
// host refuses outputs whose extent exceeds kNoOffset bytes, so a real
// output offset is never clamped away.
constexpr int kNoOffset = 0x7ffffff0;

// Buffer resource over [base, base + bytes), bytes clamped to kNoOffset.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nr = bytes > kNoOffset ? kNoOffset : static_cast<int>(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, nr, 0x00020000);
}

constexpr int kNt = 2;  // buffer cache policy: non-temporal (weights are read once)

template <int GPC>
__device__ __forceinline__ void load_groups_buf(__amdgpu_buffer_rsrc_t r, int off, bool vec, uint32_t* out) {
  if constexpr (GPC == 1) {
    out[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNt);
  } else if constexpr (GPC == 2) {
    if (vec) {
      out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kNt);
    } else {
      out[0] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kNt)) |
               (static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off + 2, 0, kNt)) << 16);
    }
  } else {
    static_assert(GPC == 4, "groups per chunk");
    if (vec) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNt);
      out[0] = v.x;
      out[1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        out[i] = static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * i, 0, kNt)) |
                 (static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off + 4 * i + 2, 0, kNt)) << 16);
    }
  }
}

// Output column of weight row `row` under the call's column map.
// (constant indices only, so a Params copy can live in registers)
template <class PT>
__device__ __forceinline__ int64_t mapped_column(PT& p, int row) {
  int64_t d = p.seg_delta[0];
#pragma unroll
  for (int sg = 1; sg < kMaxSeg; ++sg)
    if (sg < p.nseg && row >= p.seg_row0[sg]) d = p.seg_delta[sg];
  return row + d;
}

// The fast row product for block bx of gx blocks (tiles bx, bx + gx, ...).
// Shared arrays come from the calling kernel so that several bodies can be
// inlined into one fused-stack kernel without their LDS adding up.  PT is
// the kernel's own by-value Params, or a fused stack's run read in place in
// the argument segment (KParams).
template <int B, int G, int MB, bool STAGE, class PT>
__device__ __forceinline__ void fast_body(PT& p, const int bx, const int gx, unsigned char* smem,
                                          int* s_list, int* s_wave_cnt, int* s_xrow, int64_t* s_yoff) {
  constexpr int PPC = Geo<B>::PPC, CPC = Geo<B>::CPC;
  constexpr int WPC = 4 * PPC;                      // words per chunk
  constexpr int CB = 16 * PPC;                      // bytes per chunk
  constexpr int EU = CPC < G ? CPC : G;             // codes per epilogue unit
  constexpr int NEU = CPC / EU;                     // epilogue units (groups) per chunk
  constexpr int EUW = EU * B / 32;                  // words per epilogue unit
  constexpr int XP = EU / 8;                        // 16-byte activation pieces per unit
  constexpr int SW = NEU >= 2 ? NEU / 2 : 1;        // packed scale words per chunk
  constexpr int R = FastRows<B, MB>::v;
  constexpr int GSPAN = NEU >= 2 ? NEU : 1;         // groups read per chunk

  const int nchunks = p.nchunks;
  // LDS: x pieces [MB][NEU][XP][nchunks] x 16 B, unit sums [MB][NEU][nchunks],
  // then (STAGE) one staging buffer of R*PPC*64 pieces per wave.
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + static_cast<size_t>(MB) * NEU * XP * nchunks * 16);
  unsigned char* stage_all = smem + static_cast<size_t>(MB) * NEU * nchunks * (XP * 16 + 4);

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lpr = p.lpr;
  const int slot = lane / lpr;
  const int li = lane % lpr;
  const int slots_per_wave = kWave / lpr;
  const int wave_rows = slots_per_wave * R;
  const int tile_rows = kWaves * wave_rows;
  const int cpl = p.cpl;
  const bool vec = p.vec_groups != 0;
  u32x4* stage = reinterpret_cast<u32x4*>(stage_all) + wv * (R * PPC * kWave);
  const uint32_t* stage32 = reinterpret_cast<const uint32_t*>(stage);

  int expert = 0;
  int total = p.m;
  if (p.indexed) {
    expert = blockIdx.y;
    total = build_route_list(p.idx, p.m * p.slots, expert, s_list, s_wave_cnt);
    if (total == 0) return;
  }
  const int n = static_cast<int>(p.n);
  const int64_t row_bytes = p.wpr * 4;
  const int gpr2 = static_cast<int>(p.gpr) * 2;     // scale bytes per row
  const unsigned char* wexp = reinterpret_cast<const unsigned char*>(p.w) + static_cast<int64_t>(expert) * p.n * row_bytes;
  const unsigned char* sexp = reinterpret_cast<const unsigned char*>(p.scales) + static_cast<int64_t>(expert) * p.n * gpr2;
  const unsigned char* bexp = reinterpret_cast<const unsigned char*>(p.biases) + static_cast<int64_t>(expert) * p.n * gpr2;
  const int my_tiles = bx < p.tiles ? (p.tiles - 1 - bx) / gx + 1 : 0;
  const int steps = my_tiles * cpl;
  // y as one buffer resource: lanes with nothing to store aim past its end
  const __amdgpu_buffer_rsrc_t yres = make_rsrc(p.y, p.y_bytes);

  for (int c0 = 0; c0 < total; c0 += MB) {
    const int mcount = min(MB, total - c0);
    // One-row windows with chunks of at most 64 codes keep the lane's
    // activations in registers across steps (refreshed only when the chunk
    // column changes, i.e. never when a lane owns one chunk per row).
    constexpr bool XH = (MB == 1) && (CPC <= 64);
    uint32_t xh[XH ? NEU : 1][XH ? EU / 2 : 1];
    float Xh[XH ? NEU : 1];
    auto load_xh = [&](int j) {
      if constexpr (XH) {
        const int c = li + lpr * j;
#pragma unroll
        for (int e = 0; e < NEU; ++e) {
#pragma unroll
          for (int pc = 0; pc < XP; ++pc) {
            const u32x4 v = xs[(e * XP + pc) * nchunks + c];
            xh[e][4 * pc] = v.x;
            xh[e][4 * pc + 1] = v.y;
            xh[e][4 * pc + 2] = v.z;
            xh[e][4 * pc + 3] = v.w;
          }
          Xh[e] = xsum[e * nchunks + c];
        }
      }
    };
    struct Stage {
      uint32_t w[R * WPC];
      uint32_t s[R][SW];
      uint32_t b[R][SW];
    };
    // step -> (tile, chunk column j); the wave's rows are
    // [wrow0, wrow0 + wave_rows), lane (slot, li) owns rows wrow0 + r*S + slot
    auto load_stage = [&](Stage& st, int step) {
      const int i = step / cpl, j = step - (step / cpl) * cpl;
      const int tile = bx + i * gx;
      const int wrow0 = tile * tile_rows + wv * wave_rows;
      const __amdgpu_buffer_rsrc_t wr = make_rsrc(wexp + wrow0 * row_bytes, (n - wrow0) * row_bytes);
      const __amdgpu_buffer_rsrc_t sr = make_rsrc(sexp + static_cast<int64_t>(wrow0) * gpr2,
                                                  static_cast<int64_t>(n - wrow0) * gpr2);
      const __amdgpu_buffer_rsrc_t br = make_rsrc(bexp + static_cast<int64_t>(wrow0) * gpr2,
                                                  static_cast<int64_t>(n - wrow0) * gpr2);
      const int c = li + lpr * j;
      if constexpr (STAGE) {
        // piece P = lane + 64*t of the wave's chunk column: segment (row)
        // P / (lpr*PPC), piece within it P % (lpr*PPC)
        const int seg_pieces = lpr * PPC;
#pragma unroll
        for (int t = 0; t < R * PPC; ++t) {
          const int P = lane + kWave * t;
          const int sg = P / seg_pieces, within = P - sg * seg_pieces;
          const int off = static_cast<int>(sg * row_bytes) + (lpr * j) * CB + within * 16;
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, kNt);
          st.w[4 * t] = v.x;
          st.w[4 * t + 1] = v.y;
          st.w[4 * t + 2] = v.z;
          st.w[4 * t + 3] = v.w;
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int sg = r * slots_per_wave + slot;
        if constexpr (!STAGE) {
#pragma unroll
          for (int pp = 0; pp < PPC; ++pp) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
                wr, static_cast<int>(sg * row_bytes) + c * CB + pp * 16, 0, kNt);
            st.w[r * WPC + 4 * pp] = v.x;
            st.w[r * WPC + 4 * pp + 1] = v.y;
            st.w[r * WPC + 4 * pp + 2] = v.z;
            st.w[r * WPC + 4 * pp + 3] = v.w;
          }
        }
        const int goff = sg * gpr2 + ((c * CPC) / G) * 2;
        load_groups_buf<GSPAN>(sr, goff, vec, st.s[r]);
        load_groups_buf<GSPAN>(br, goff, vec, st.b[r]);
      }
    };

    float acc[R][MB];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mi = 0; mi < MB; ++mi) acc[r][mi] = 0.0f;

    auto compute_stage = [&](const Stage& st, int step) {
      const int i = step / cpl, j = step - (step / cpl) * cpl;
      const int c = li + lpr * j;
      if constexpr (XH) {
        if (cpl > 1) load_xh(j);
      }
      if constexpr (STAGE) {
        // hand the pieces over: lane order in, chunk order out
#pragma unroll
        for (int t = 0; t < R * PPC; ++t) {
          u32x4 v;
          v.x = st.w[4 * t];
          v.y = st.w[4 * t + 1];
          v.z = st.w[4 * t + 2];
          v.w = st.w[4 * t + 3];
          stage[lane + kWave * t] = v;
        }
      }
#pragma unroll
      for (int e = 0; e < NEU; ++e) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          // cut this row's codes of the unit once, for every window row
          uint32_t wu[EUW];
          if constexpr (STAGE) {
            const int sg = r * slots_per_wave + slot;
            const int base = (sg * lpr + li) * WPC + e * EUW;
#pragma unroll
            for (int h = 0; h < EUW; ++h) wu[h] = stage32[base + h];
          } else {
#pragma unroll
            for (int h = 0; h < EUW; ++h) wu[h] = st.w[r * WPC + e * EUW + h];
          }
          uint32_t q[EU / 2];
          unpack_codes<B, EU>(wu, q);
          const float sv = group_value<GSPAN>(st.s[r], e);
          const float bv = group_value<GSPAN>(st.b[r], e);
#pragma unroll
          for (int mi = 0; mi < MB; ++mi) {
            if (mi < mcount) {
              uint32_t xv[EU / 2];
              float X;
              if constexpr (XH) {
#pragma unroll
                for (int pp = 0; pp < EU / 2; ++pp) xv[pp] = xh[e][pp];
                X = Xh[e];
              } else {
#pragma unroll
                for (int pc = 0; pc < XP; ++pc) {
                  const u32x4 v = xs[((mi * NEU + e) * XP + pc) * nchunks + c];
                  xv[4 * pc] = v.x;
                  xv[4 * pc + 1] = v.y;
                  xv[4 * pc + 2] = v.z;
                  xv[4 * pc + 3] = v.w;
                }
                X = xsum[(mi * NEU + e) * nchunks + c];
              }
              float a = 0.0f;
#pragma unroll
              for (int pp = 0; pp < EU / 2; ++pp) a = dot2(q[pp], xv[pp], a);
              acc[r][mi] = __builtin_fmaf(sv, a, acc[r][mi]);
              acc[r][mi] = __builtin_fmaf(bv, X, acc[r][mi]);
            }
          }
        }
      }
      if (j == cpl - 1) {
        const int tile = bx + i * gx;
        const int wrow0 = tile * tile_rows + wv * wave_rows;
        float red[R][MB];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int mi = 0; mi < MB; ++mi) {
            red[r][mi] = lpr == 64 ? gsum<64>(acc[r][mi]) : (lpr == 32 ? gsum<32>(acc[r][mi]) : gsum<16>(acc[r][mi]));
            acc[r][mi] = 0.0f;
          }
        // lane li of a column group stores element li (+ 16, ...) of its
        // R x MB results; lanes with nothing to store aim past the buffer
#pragma unroll
        for (int e0 = 0; e0 < R * MB; e0 += 16) {
          const int e = e0 + li;
          float v = 0.0f;
#pragma unroll
          for (int k2 = e0; k2 < e0 + 16 && k2 < R * MB; ++k2) v = (e == k2) ? red[k2 / MB][k2 % MB] : v;
          const int r = e / MB, mi = e - (e / MB) * MB;
          const int row = wrow0 + r * slots_per_wave + slot;
          const bool ok = e < R * MB && li < 16 && mi < mcount && row < n;
          const int off = ok ? static_cast<int>((s_yoff[ok ? mi : 0] + mapped_column(p, row)) * 4) : kNoOffset;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(apply_epi(v, p.epi)), yres, off, 0, 0);
        }
      }
    };

    // the first step's weights are in flight while the window is staged
    Stage sa, sb;
    if (steps > 0) load_stage(sa, 0);
    if (tid < mcount) {
      const int e = c0 + tid;
      if (p.indexed) {
        const int t = s_list[e];
        const int row = t / p.slots, sl = t % p.slots;
        s_xrow[tid] = row;
        s_yoff[tid] = (static_cast<int64_t>(row) * p.slots + sl) * p.n;
      } else {
        s_xrow[tid] = e;
        s_yoff[tid] = static_cast<int64_t>(e) * p.ldy;
      }
    }
    __syncthreads();
    // ---- stage the window: activation pieces and per-unit sums ----
    for (int t = tid; t < mcount * nchunks * NEU; t += kThreads) {
      const int mi = t / (nchunks * NEU);
      const int rest = t % (nchunks * NEU);
      const int c = rest / NEU, e = rest % NEU;
      const u32x4* src = reinterpret_cast<const u32x4*>(
          p.x + static_cast<int64_t>(s_xrow[mi]) * p.k + static_cast<int64_t>(c) * CPC + e * EU);
      uint32_t xin[EU / 2];
#pragma unroll
      for (int pc = 0; pc < XP; ++pc) {
        const u32x4 v = src[pc];
        xin[4 * pc] = v.x;
        xin[4 * pc + 1] = v.y;
        xin[4 * pc + 2] = v.z;
        xin[4 * pc + 3] = v.w;
      }
      // pairs in the order the unpack pairs the codes; X over those pairs
      float X = 0.0f;
      const uint32_t ones = 0x3f803f80u;  // bf16 pair {1, 1}
#pragma unroll
      for (int pc = 0; pc < XP; ++pc) {
        u32x4 o;
        o.x = slot_pair<B>(xin, 4 * pc);
        o.y = slot_pair<B>(xin, 4 * pc + 1);
        o.z = slot_pair<B>(xin, 4 * pc + 2);
        o.w = slot_pair<B>(xin, 4 * pc + 3);
        X = dot2(o.x, ones, X);
        X = dot2(o.y, ones, X);
        X = dot2(o.z, ones, X);
        X = dot2(o.w, ones, X);
        xs[((mi * NEU + e) * XP + pc) * nchunks + c] = o;
      }
      xsum[(mi * NEU + e) * nchunks + c] = X;
    }
    __syncthreads();

    load_xh(0);
    if (steps > 0) {
      int step = 0;
      for (; step + 1 < steps; step += 2) {
        load_stage(sb, step + 1);
        compute_stage(sa, step);
        load_stage(sa, min(step + 2, steps - 1));
        compute_stage(sb, step + 1);
      }
      if (step < steps) compute_stage(sa, step);
    }
    __syncthreads();  // LDS window reused by the next chunk of routed rows
  }
}

template <int B, int G, int MB, bool STAGE>
__global__ __launch_bounds__(kThreads) void qrow_fast(const Params p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_list[kMaxList];
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_xrow[QGEMV_MAX_WINDOW];
  __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];
  fast_body<B, G, MB, STAGE>(p, blockIdx.x, gridDim.x, smem, s_list, s_wave_cnt, s_xrow, s_yoff);
}

// ---------------------------------------------------------------------------
// MFMA kernel: v_mfma_f32_16x16x32_bf16 with a block-diagonal activation
// operand.
//
// A wave owns 16 output columns and walks K in load groups of R rounds of
// 128 codes per column.  Lane l (column j = l % 16, quarter q = l / 16) owns
// units qR .. qR + R - 1 of its column's share of a group (whole 16-byte
// pieces, read from LDS once per group) and in round r holds unit qR + r as
// exact bf16 pairs in the unpack's slot order.  MFMA step s (0..3) feeds
// slots 8s..8s+7 of every lane's unit as the B operand (k-index 8q + e of
// column j).  Row i = 4m + q' of the A operand holds window row m's
// activations of unit q'R + r in k-indices 8q'..8q'+7 and zeros elsewhere,
// so after the four steps D[4m + q'][j] is the fp32 dot of unit q'R + r of
// column j with window row m, every product exact.  Lane l holds
// D[4(l/16) + q'][l % 16] for q' = 0..3 (one window row, one column, four
// units).  Per round the bias terms of the four units,
// sum over u of bias(u) * X(row, u), come first as one fp32 16x16x4 product
// accumulated into the lane's outputs; then the lane folds its units' scale
// terms in unit order, P = fma(s, D, P).  No lane reduction follows, and
// each output depends only on its own window row's activations, wherever the
// row sits in the window.
//
// Loads: a group of R rounds, R chosen so that a column's share of a group
// is L whole 128-byte lines, comes in as 16-byte pieces, each group of 8
// lanes of one load fetching one whole line (a streaming line asked for by
// two different loads is read from HBM twice).  The pieces go to registers
// one group ahead, then to a per-wave LDS slot laid out line-major
// ([line][column]) with the 8 pieces of column c's line rotated by c / 2,
// so the 16 lanes that read the same piece of 16 columns hit 16 different
// bank groups.
//
// K split: a handle may split K into S = 1, 2 or 4 consecutive parts (fixed
// at create from its shape, never from the window).  The S waves of a
// column group each fold their part's units in order from zero, and the
// parts are then added in order, P = ((P0 + P1) + P2) + P3, through the
// waves' LDS slots.
//
// Gate/up pairs: the 16 MFMA columns of a tile are rows f0..f0+7 of the gate
// matrix (columns 0-7) and the same rows of the up matrix (columns 8-15).
// Even loads of a group fetch only columns 0-7 and odd loads only 8-15, so
// each load reads one matrix.  Every column keeps the arithmetic it has in
// a plain call; at the tile's end lane j + 8 hands its up value to lane j
// (DPP row rotate by 8), which stores silu(g) * u for output column f0 + j.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 128-code rounds per load group: the fewest whose codes end on a byte.
__host__ __device__ constexpr int group_rounds(int b) {
  return b == 8 ? 1 : (b == 4 ? 2 : ((b == 2 || b == 6) ? 4 : 8));
}
// Load groups per pipeline stage of the kernels that hand out units in the
// block: 2 for 2-, 4- and 8-bit codes, whose groups are one 128-byte line a
// column (2 KiB a wave).  A stage's groups are loaded together and computed
// one after the other in order, so a wave keeps twice the bytes in flight
// while it computes and the arithmetic is the tile walk's.
__host__ __device__ constexpr int dyn_stage_groups(int b) { return (b == 2 || b == 4 || b == 8) ? 2 : 1; }
// LDS bytes of one wave's load-group slot: 16 columns' weights (R*B/8 lines
// of 128 bytes each) and their scales and biases (rows of 32 bytes padded to 48).
__host__ __device__ constexpr int group_slot(int b, int g) {
  const int r = group_rounds(b), sb = 256 * r / g, sbp = sb < 4 ? 4 : sb;
  return 16 * (r * b / 8) * 128 + 2 * 16 * (sbp % 32 == 0 ? sbp + 16 : sbp);
}

template <int B, int G> struct MGroup {
  static constexpr int R = group_rounds(B);        // rounds per group
  static constexpr int L = R * B / 8;              // 128-byte lines per column per group
  static constexpr int WLD = 2 * L;                // 16-byte weight loads per lane per group
  static constexpr int SB = 256 * R / G;           // scale bytes per column per group
  static constexpr bool S16 = SB % 16 == 0;        // scales as 16-byte pieces, else dwords
  static constexpr int SBP = SB < 4 ? 4 : SB;      // bytes kept per column (the aligned dword when 2)
  static constexpr int SSZ = S16 ? 16 : 4;         // bytes of one scale load
  static constexpr int SLANES = 16 * SBP / SSZ;    // lanes of one scale load
  static constexpr int SSTR = SBP % 32 == 0 ? SBP + 16 : SBP;   // LDS bytes per column of scales
  static constexpr int WBYTES = 16 * L * 128;
  static constexpr int SLOT = WBYTES + 2 * 16 * SSTR;
  static_assert(R * B % 8 == 0 && SLANES <= 64 && SLOT == group_slot(B, G), "group geometry");
};

// Waves per block of the kernels that hand out units in the block (the
// whole CU's share of a large matrix in one block): as many as both the
// register share and the LDS allow.
// * Registers: 3 waves a SIMD (168 VGPRs) for windows of up to 8 rows, but 2
//   (8 waves) for the 5-bit bodies that need more; at 16 rows 11 (3 waves on
//   three SIMDs, 2 on the fourth), or 8 for 3- and 5-bit codes.
// * LDS at K = 2048: the staged window, the zero area and the unit sums, as
//   the host plans them, plus one group slot a wave.  At 16 rows the window
//   takes 64 KiB, which leaves room for 8 slots of 3-bit or 5-bit/128 codes
//   and only 7 of 5-bit codes in groups of 32 or 64.
// At larger K the host finds the plan too large and takes the tile walk.
__host__ __device__ constexpr int dyn_waves(int b, int g, int mb, bool wide) {
  const bool big = b == 5 && (wide ? (g <= 64 && mb >= 2 && mb <= 8) : (g == 32 || mb == 8));
  const int regs = mb < 16 ? (big ? 8 : 12) : ((b == 3 || b == 5) ? 8 : 11);
  const int units = 2048 / 32;
  const int fixed = mb * (units * 64 + 16) + 256 * group_rounds(b) + mb * (units + 4) * 4;
  const int lds = (static_cast<int>(kMaxMfmaLds) - fixed) / group_slot(b, g);
  return regs < lds ? regs : lds;
}
template <int B, int G, int MB, bool WIDE> struct DynWaves {
  static constexpr int v = dyn_waves(B, G, MB, WIDE);
  static_assert(v >= 4, "a unit-handout block holds at least one wave a SIMD");
};

// Waves per block: a wide window's activations are staged once for 8 waves.
template <int MB> struct MWaves {
  static constexpr int v = MB >= 8 ? 8 : 4;
};

// 4 x 4 transpose of W-dword items across the four 16-lane rows of a wave.
// On entry the lanes of row q hold items X_q[0..3] in q[W*t .. W*t+W-1]; on
// exit they hold X_0[q], X_1[q], X_2[q], X_3[q].  First the rows two apart swap
// (permlane32: the upper 32 lanes of the first operand with the lower 32 of
// the second), then adjacent rows (permlane16: the odd rows of the first
// operand with the even rows of the second).
template <int W, bool ROWS_TWO_APART = true>
__device__ __forceinline__ void transpose_items(uint32_t* q) {
  if constexpr (ROWS_TWO_APART) {
#pragma unroll
    for (int d = 0; d < W; ++d) {
      const auto a = __builtin_amdgcn_permlane32_swap(q[d], q[2 * W + d], false, false);
      q[d] = a[0];
      q[2 * W + d] = a[1];
      const auto b = __builtin_amdgcn_permlane32_swap(q[W + d], q[3 * W + d], false, false);
      q[W + d] = b[0];
      q[3 * W + d] = b[1];
    }
  }
#pragma unroll
  for (int d = 0; d < W; ++d) {
    const auto a = __builtin_amdgcn_permlane16_swap(q[d], q[W + d], false, false);
    q[d] = a[0];
    q[W + d] = a[1];
    const auto b = __builtin_amdgcn_permlane16_swap(q[2 * W + d], q[3 * W + d], false, false);
    q[2 * W + d] = b[0];
    q[3 * W + d] = b[1];
  }
}
__device__ __forceinline__ void transpose_rows(uint32_t* q) { transpose_items<4>(q); }

// t = mi * units + un for 0 <= t < 2^22: the quotient from one fp32 product
// with the rounded reciprocal is off by at most one (relative error below
// 2^-22 on a quotient below 2^22), and one correction step fixes it.
// (Selects, not branches: it sits ahead of a kernel's first loads.)
__device__ __forceinline__ void split_units(int t, int units, float inv_units, int& mi, int& un) {
  const int q = static_cast<int>(static_cast<float>(t) * inv_units);
  const int r = t - q * units;
  const int fix = r < 0 ? -1 : (r >= units ? 1 : 0);
  mi = q + fix;
  un = r - fix * units;
}

// WIDE selects the wide-window form: after the unpack, the four lanes of a
// column trade quarters of their units (transpose_rows), so that lane (j, q)
// holds k-quarter q of all four units of the round; each unit is then one
// 16x16x32 product over every window row at once (A row i = window row i),
// and lane (j, q) folds window rows 4q .. 4q+3 of column j.
template <int B, int G, int MB, bool WIDE = false, bool GU = false, bool IDX = false, bool DYN = false,
          class PT = const Params, int NWO = 0>
__device__ __forceinline__ void mfma_body(PT& p, const int bx, const int gx, unsigned char* smem,
                                          int* s_wave_cnt, int* s_xrow, int64_t* s_yoff, int* s_next = nullptr) {
  static_assert(!DYN || (!GU && !IDX), "units handed out in a block: plain and strided calls");
  using MG = MGroup<B, G>;
  constexpr int R = MG::R, SSZ = MG::SSZ;
  constexpr int NG = DYN ? dyn_stage_groups(B) : 1;   // load groups per stage
  // a two-group stage whose groups' scales are dwords (4 or 8 bytes a column)
  // loads both groups' scales (and biases) of a column at once: 8 or 16
  // bytes from an even group, by lanes 0-15 (lane = column)
  constexpr bool CS = NG == 2 && MG::SSZ == 4 && MG::SB >= 4;
  constexpr int CW = CS ? MG::SB / 2 : 1;             // dwords of a column's two groups
  static_assert(!CS || !GU, "combined scale loads: plain and strided calls");
  constexpr int NW = DYN ? DynWaves<B, G, MB, WIDE>::v : (NWO ? NWO : MWaves<MB>::v), NT = NW * kWave;
  constexpr int NMB = (MB + 3) / 4;         // 4-row blocks of the window
  // outputs each lane folds: one per 4-row block, or (wide form) window rows
  // 4q .. 4q+3 of its column, as many as the window can hold
  constexpr int NACC = WIDE ? (MB < 4 ? MB : 4) : NMB;
  constexpr int ZB = R * 256;               // zero area: one group's activations

  // the call's shape as the host derived it: no division on the device
  // before the first loads (each instruction of a lone wave costs about 4
  // cycles, and a small call's waves run alone on their SIMDs)
  const int units = static_cast<int>(p.k) >> 5;
  const int ksh = p.ks_shift;
  const int S = 1 << ksh;                   // K-parts per column
  const int gpp = p.gpp;                    // groups per K-part
  const int ncg = NW >> ksh;                // column groups (of 16 columns) per block
  const float inv_units = p.inv_units;
  const int tiles = p.tiles;
  const int mrows = IDX ? MB : min(p.m, MB);       // window rows staged
  const int xstride = units * 64 + 16;                     // bytes per staged row
  const int sstride = units + 4;                           // floats per row of unit sums
  // LDS: activations [mrows][units][32 slots] bf16, a zero area of one
  // group's activations (the A operand of lanes outside the block diagonal,
  // read at the same offsets as a live lane's), unit sums [mrows][units]
  // fp32 (rows of activations and of sums padded by 16 bytes, so the rows a
  // wave reads at once fall in different banks), the routed list (indexed
  // calls), one slot per wave.  With a K split, each wave's partial sums
  // [NACC][64 lanes] fp32 go to the start of its own slot at a tile's end:
  // the slot's last group has been read by then (a wave's LDS operations
  // stay in order), and the next hand-off into it follows the barrier after
  // the partials are read.
  unsigned char* zero_area = smem + static_cast<size_t>(mrows) * xstride;
  float* xsum = reinterpret_cast<float*>(zero_area + ZB);
  int* s_list = reinterpret_cast<int*>(xsum + static_cast<size_t>(mrows) * sstride);
  unsigned char* slots = reinterpret_cast<unsigned char*>(s_list + (IDX ? kMaxList : 0));

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wv = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane % 16, qd = lane / 16;
  const int cg = wv >> ksh, ks = wv & (S - 1);    // column group, K-part
  unsigned char* slot = slots + static_cast<size_t>(wv) * MG::SLOT;
  static_assert(4 * kWave * 4 <= MG::SLOT, "partial sums fit a slot");

  int expert = 0;
  int total = p.m;
  if (IDX) {
    expert = blockIdx.y;
    total = build_route_list<NT>(p.idx, p.m * p.slots, expert, s_list, s_wave_cnt);
    if (total == 0) return;
  }
  const int n = static_cast<int>(p.n);
  const int64_t row_bytes = p.wpr * 4;
  const int gpr2 = static_cast<int>(p.gpr) * 2;
  const unsigned char* wexp = reinterpret_cast<const unsigned char*>(p.w) + static_cast<int64_t>(expert) * p.n * row_bytes;
  const unsigned char* sexp = reinterpret_cast<const unsigned char*>(p.scales) + static_cast<int64_t>(expert) * p.n * gpr2;
  const unsigned char* bexp = reinterpret_cast<const unsigned char*>(p.biases) + static_cast<int64_t>(expert) * p.n * gpr2;
  // gate/up pairing is compiled in or out: as a run-time flag its pointers
  // and descriptors held scalar registers in every kernel
  constexpr bool gu = GU;
  const int cw = gu ? 8 : 16;                 // output columns per column group
  const unsigned char* wexp2 = gu ? reinterpret_cast<const unsigned char*>(p.w2) + static_cast<int64_t>(expert) * p.n * row_bytes : wexp;
  const unsigned char* sexp2 = gu ? reinterpret_cast<const unsigned char*>(p.scales2) + static_cast<int64_t>(expert) * p.n * gpr2 : sexp;
  const unsigned char* bexp2 = gu ? reinterpret_cast<const unsigned char*>(p.biases2) + static_cast<int64_t>(expert) * p.n * gpr2 : bexp;

  // ---- per-lane constants of the loads and reads (the same for every group) ----
  // weight load t: lanes 8a..8a+7 fetch line lam = 8t + a of the slot, which
  // is line lam / 16 of column lam % 16's share; lane 8a + e brings piece
  // (e - c/2) mod 8 of it, so piece pp of column c's line sits at e = (pp + c/2) mod 8
  int w_voff[MG::WLD];
#pragma unroll
  for (int t = 0; t < MG::WLD; ++t) {
    const int lam = 8 * t + lane / 8, c = lam % 16, ln = lam / 16;
    const int pp = (lane % 8 - c / 2) & 7;
    const int row = gu ? (c & 7) : c;         // row of its matrix within the tile
    w_voff[t] = static_cast<int>(row * row_bytes) + ln * 128 + pp * 16;
  }
  // scale (bias) load: lane L < SLANES brings piece (or dword) L % per of
  // column L / per, per = SBP / SSZ
  constexpr int SPER = MG::SBP / SSZ;
  const bool s_live = lane < MG::SLANES;
  const int s_col = lane / SPER;
  const int s_voff = (gu ? (s_col & 7) : s_col) * gpr2 + (lane % SPER) * SSZ;
  const int s_woff = (lane / SPER) * MG::SSTR + (lane % SPER) * SSZ;   // its place in the slot
  // Lane (j, qd) owns units qd*R .. qd*R + R - 1 of column j's share of a
  // group (unit qd*R + r in round r): NP = R*B/4 whole 16-byte pieces,
  // pieces qd*NP + t of the share, at line (qd*NP + t) / 8, piece
  // (qd*NP + t) % 8 of the slot (rotated by j / 2).
  constexpr int NP = R * B / 4;
  static_assert((R * B) % 4 == 0, "a lane's units are whole pieces");
  // (set once the window is staged: only the hand-off reads need them)
  int p_off[NP];
  const int s_off = MG::WBYTES + j * MG::SSTR;
  const int b_off = s_off + 16 * MG::SSTR;
  constexpr int UPG = G / 32;                 // units per group

  // A step is one group of this wave's K-part of one tile; cursors walk the
  // steps in order: tiles bx, bx + gx, ... below the tile count, and in each
  // the K-part's groups (gr counts groups from the start of the row)
  struct Cursor {
    int tile, gr, k;   // k: units taken so far (units handed out in the block)
  };
  const int gr0 = ks * gpp;
  // Units handed out in the block (DYN, calls with no K split): the
  // block owns 16-column units [u0, u1); each wave takes its first two
  // statically (u0 + wave, u0 + NW + wave) and then the next free one from
  // an LDS counter, so faster waves take more and the block's waves end
  // together.  A column's arithmetic does not depend on its wave.
  int u0 = 0, u1 = 0;
  if constexpr (DYN) {
    u0 = static_cast<int>(static_cast<int64_t>(bx) * tiles / gx);
    u1 = static_cast<int>(static_cast<int64_t>(bx + 1) * tiles / gx);
  }
  const int tend = DYN ? u1 : tiles;   // a cursor is past the end at tile >= tend
  auto next_unit = [&](Cursor& c) -> int {
    ++c.k;
    if (c.k == 1) return u0 + NW + wv;
    if (c.tile >= u1) return u1;
    int u = 0;
    if (lane == 0) u = atomicAdd(s_next, 1);
    return __builtin_amdgcn_readfirstlane(u);
  };
  auto advance = [&](Cursor& c) {
    c.gr += NG;
    if (c.gr == gr0 + gpp) {
      c.gr = gr0;
      if constexpr (DYN) {
        c.tile = next_unit(c);
      } else {
        c.tile += gx;
      }
    }
  };
  struct Stage {
    u32x4 w[NG][MG::WLD];
    uint32_t s[NG][SSZ / 4];
    uint32_t b[NG][SSZ / 4];
    uint32_t cs[CW], cb[CW];   // both groups' scales and biases of column lane (CS)
    Cursor cur;   // the step these loads belong to (its first group)
  };
  // a step's loads into registers (past the last step: loads that read nothing)
  auto load_stage = [&](Stage& sg, const Cursor& c) {
    sg.cur = c;
    const bool real = c.tile < tend;
    const int c0 = DYN ? c.tile * 16 : (c.tile * ncg + cg) * cw;
    const int ncols = real ? n - c0 : 0;
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wexp + static_cast<int64_t>(c0) * row_bytes,
                                                static_cast<int64_t>(ncols) * row_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(sexp + static_cast<int64_t>(c0) * gpr2,
                                                static_cast<int64_t>(ncols) * gpr2);
    const __amdgpu_buffer_rsrc_t br = make_rsrc(bexp + static_cast<int64_t>(c0) * gpr2,
                                                static_cast<int64_t>(ncols) * gpr2);
    // the up matrix's rows of the same tile (gate/up pairs only)
    const __amdgpu_buffer_rsrc_t wr2 = make_rsrc(wexp2 + static_cast<int64_t>(c0) * row_bytes,
                                                 static_cast<int64_t>(gu ? ncols : 0) * row_bytes);
    // the stage's groups: weights, then scales, of each in order
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2) {
      const int gr = c.gr + g2;
      const int wsoff = gr * (MG::L * 128);
#pragma unroll
      for (int t = 0; t < MG::WLD; ++t)
        sg.w[g2][t] = __builtin_amdgcn_raw_buffer_load_b128((t & 1) && gu ? wr2 : wr, w_voff[t], wsoff, kNt);
      // this group's scales: SB bytes per column from byte gr*SB of the row
      // (at SB = 2, the aligned dword that holds them); default cache policy,
      // since a row's scale line serves several groups.  A gate/up tile loads
      // its gate columns and its up columns separately (a lane outside a
      // load's range reads zeros), and merges them.
      const int ssoff = MG::SB < 4 ? ((gr * MG::SB) & ~3) : gr * MG::SB;
      const int sv = s_live && !(gu && s_col >= 8) ? s_voff : kNoOffset;
      if constexpr (CS) {
        if (g2 == 0) {
          const int cv = lane < 16 ? lane * gpr2 : kNoOffset;
          if constexpr (CW == 4) {
            const u32x4 a4 = __builtin_amdgcn_raw_buffer_load_b128(sr, cv, ssoff, 0);
            const u32x4 b4 = __builtin_amdgcn_raw_buffer_load_b128(br, cv, ssoff, 0);
            sg.cs[0] = a4.x; sg.cs[1] = a4.y; sg.cs[2] = a4.z; sg.cs[3] = a4.w;
            sg.cb[0] = b4.x; sg.cb[1] = b4.y; sg.cb[2] = b4.z; sg.cb[3] = b4.w;
          } else {
            const u32x2 a2 = __builtin_amdgcn_raw_buffer_load_b64(sr, cv, ssoff, 0);
            const u32x2 b2 = __builtin_amdgcn_raw_buffer_load_b64(br, cv, ssoff, 0);
            sg.cs[0] = a2.x; sg.cs[1] = a2.y;
            sg.cb[0] = b2.x; sg.cb[1] = b2.y;
          }
        }
      } else if constexpr (SSZ == 16) {
        u32x4 a4 = __builtin_amdgcn_raw_buffer_load_b128(sr, sv, ssoff, 0);
        u32x4 b4 = __builtin_amdgcn_raw_buffer_load_b128(br, sv, ssoff, 0);
        if (gu) {
          const __amdgpu_buffer_rsrc_t sr2 = make_rsrc(sexp2 + static_cast<int64_t>(c0) * gpr2,
                                                       static_cast<int64_t>(ncols) * gpr2);
          const __amdgpu_buffer_rsrc_t br2 = make_rsrc(bexp2 + static_cast<int64_t>(c0) * gpr2,
                                                       static_cast<int64_t>(ncols) * gpr2);
          const int sv2 = s_live && s_col >= 8 ? s_voff : kNoOffset;
          a4 |= __builtin_amdgcn_raw_buffer_load_b128(sr2, sv2, ssoff, 0);
          b4 |= __builtin_amdgcn_raw_buffer_load_b128(br2, sv2, ssoff, 0);
        }
        sg.s[g2][0] = a4.x; sg.s[g2][1] = a4.y; sg.s[g2][2] = a4.z; sg.s[g2][3] = a4.w;
        sg.b[g2][0] = b4.x; sg.b[g2][1] = b4.y; sg.b[g2][2] = b4.z; sg.b[g2][3] = b4.w;
      } else {
        sg.s[g2][0] = __builtin_amdgcn_raw_buffer_load_b32(sr, sv, ssoff, 0);
        sg.b[g2][0] = __builtin_amdgcn_raw_buffer_load_b32(br, sv, ssoff, 0);
        if (gu) {
          const __amdgpu_buffer_rsrc_t sr2 = make_rsrc(sexp2 + static_cast<int64_t>(c0) * gpr2,
                                                       static_cast<int64_t>(ncols) * gpr2);
          const __amdgpu_buffer_rsrc_t br2 = make_rsrc(bexp2 + static_cast<int64_t>(c0) * gpr2,
                                                       static_cast<int64_t>(ncols) * gpr2);
          const int sv2 = s_live && s_col >= 8 ? s_voff : kNoOffset;
          sg.s[g2][0] |= __builtin_amdgcn_raw_buffer_load_b32(sr2, sv2, ssoff, 0);
          sg.b[g2][0] |= __builtin_amdgcn_raw_buffer_load_b32(br2, sv2, ssoff, 0);
        }
      }
    }
  };

  // this lane's outputs: element i is window row 4i + qd (4-row blocks) or
  // 4qd + i (wide form) of column j; elements past NACC are never stored
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int mcount = 0;

  // Bias terms: a round's sum over its four units of bias(u) * X(row, u)
  // is one fp32 16x16x4 product, X [16 rows][4 units] times bias [4 units]
  // [16 columns], accumulated straight into acc.  Its A row rho carries the
  // window row that lands in the element of acc that folds that row: rho
  // itself in the wide form, 4 (rho % 4) + rho / 4 for 4-row blocks.
  const int ai = lane % 16;
  const int xrow = WIDE ? ai : 4 * (ai % 4) + ai / 4;
  // bias of unit qd*R + r of column j, from the slot's bias bytes: group
  // (qd*R + r) / UPG of the share, = qd*R/UPG + r/UPG when UPG divides R,
  // else qd*R/UPG (r < R <= UPG/2 never crosses a group)
  const int b_lane = ((qd * R) / UPG) * 2;

  // per-lane LDS offsets (from smem) of the A operands, set for each pass of
  // window rows and advanced per group
  int a_base[NMB], a_live[NMB], xa_base = 0;
  auto set_bases = [&]() {
    xa_base = mrows * xstride + ZB + ((xrow < mcount ? xrow : 0) * sstride + qd * R) * 4;
    if constexpr (WIDE) {
      // A operand of lane (row ai, k-quarter qd): quarter qd of each unit of
      // window row ai (rows past the window read row 0 and are never stored)
      a_base[0] = (ai < mcount ? ai : 0) * xstride + qd * 16;
      a_live[0] = 1;
    } else {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const int am = 4 * mb + ai / 4;
        // lane (row ai, k-quarter qd) is live when its quarter is its row's
        // unit and the window row exists
        const bool live = (qd == ai % 4) && (am < mcount);
        a_live[mb] = live ? 1 : 0;
        a_base[mb] = live ? am * xstride + qd * R * 64 : mrows * xstride;
      }
    }
  };

  auto compute_group = [&](const u32x4 (&gw)[MG::WLD], const uint32_t (&gs)[SSZ / 4], const uint32_t (&gb)[SSZ / 4],
                           const uint32_t* cs, const uint32_t* cb, const Cursor& c, const int gr) {
    // hand the group over: lane order in, the slot layout out (the wave's
    // previous reads of the slot precede these writes in its LDS queue)
#pragma unroll
    for (int t = 0; t < MG::WLD; ++t) reinterpret_cast<u32x4*>(slot)[t * kWave + lane] = gw[t];
    if constexpr (CS) {
      // this group's half of column lane's scales and biases (SSTR = SB here)
      if (lane < 16) {
        if constexpr (CW == 4) {
          u32x2 a2, b2;
          a2.x = cs[0]; a2.y = cs[1];
          b2.x = cb[0]; b2.y = cb[1];
          *reinterpret_cast<u32x2*>(slot + MG::WBYTES + lane * MG::SSTR) = a2;
          *reinterpret_cast<u32x2*>(slot + MG::WBYTES + 16 * MG::SSTR + lane * MG::SSTR) = b2;
        } else {
          *reinterpret_cast<uint32_t*>(slot + MG::WBYTES + lane * MG::SSTR) = cs[0];
          *reinterpret_cast<uint32_t*>(slot + MG::WBYTES + 16 * MG::SSTR + lane * MG::SSTR) = cb[0];
        }
      }
    } else if (s_live) {
      if constexpr (SSZ == 16) {
        u32x4 a4, b4;
        a4.x = gs[0]; a4.y = gs[1]; a4.z = gs[2]; a4.w = gs[3];
        b4.x = gb[0]; b4.y = gb[1]; b4.z = gb[2]; b4.w = gb[3];
        *reinterpret_cast<u32x4*>(slot + MG::WBYTES + s_woff) = a4;
        *reinterpret_cast<u32x4*>(slot + MG::WBYTES + 16 * MG::SSTR + s_woff) = b4;
      } else {
        *reinterpret_cast<uint32_t*>(slot + MG::WBYTES + s_woff) = gs[0];
        *reinterpret_cast<uint32_t*>(slot + MG::WBYTES + 16 * MG::SSTR + s_woff) = gb[0];
      }
    }
    int a_grp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) a_grp[mb] = a_base[mb] + a_live[mb] * (gr * R * 256);
    const int xa_grp = xa_base + gr * R * 16;
    // the group's scale bytes of column j (the kept bytes), read once
    constexpr int NSW = MG::SBP / 4;
    uint32_t sw[NSW];
    if constexpr (MG::SBP >= 16) {
#pragma unroll
      for (int t = 0; t < MG::SBP / 16; ++t) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(slot + s_off + t * 16);
        sw[4 * t] = v.x;
        sw[4 * t + 1] = v.y;
        sw[4 * t + 2] = v.z;
        sw[4 * t + 3] = v.w;
      }
    } else if constexpr (MG::SBP == 8) {
      const u32x2 v = *reinterpret_cast<const u32x2*>(slot + s_off);
      sw[0] = v.x;
      sw[1] = v.y;
    } else {
      sw[0] = *reinterpret_cast<const uint32_t*>(slot + s_off);
    }
    u32x4 pcs[NP];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // this round's unit (words rB .. rB + B - 1 of the lane's pieces): read
      // the pieces the previous round has not
#pragma unroll
      for (int t = 0; t < NP; ++t)
        if (t >= (r * B) / 4 && t <= (r * B + B - 1) / 4 && (r == 0 || t > ((r - 1) * B + B - 1) / 4))
          pcs[t] = *reinterpret_cast<const u32x4*>(slot + p_off[t]);
      uint32_t wu[B];
#pragma unroll
      for (int h = 0; h < B; ++h) wu[h] = pcs[(r * B + h) / 4][(r * B + h) % 4];
      // scales of the round's four units i*R + r; at SB = 2 the round's one
      // group is a half of the aligned dword
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int si = MG::SB < 4 ? ((gr * R + r) & 1) : (i * R + r) / UPG;
        const uint32_t w = sw[MG::SB < 4 ? 0 : si / 2];
        sv[i] = (si & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
      }
      // the bias of this lane's unit qd*R + r
      const int bofs = MG::SB < 4 ? ((gr * R + r) & 1) * 2 : (UPG <= R ? (r / UPG) * 2 : 0);
      {
        const float xa = *reinterpret_cast<const float*>(smem + xa_grp + r * 4);
        const uint32_t braw = *reinterpret_cast<const uint16_t*>(slot + b_off + b_lane + bofs);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, __uint_as_float(braw << 16), acc, 0, 0, 0);
      }
      if constexpr (WIDE) {
        // A operand: quarter qd of the round's four units of row lane % 16;
        // the unit sums of the rows this lane folds
        u32x4 aw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) aw[u] = *reinterpret_cast<const u32x4*>(smem + a_grp[0] + (u * R + r) * 64);
        // B operand: this lane's unit as 16 exact bf16 pairs, then quarter
        // qd of each of the four units
        uint32_t qp[16];
        if constexpr (B == 4 || B == 8) {
          // a quarter of a unit is whole words (8 codes in 1 or 2 words,
          // each unpacked on its own): trade the packed words, then unpack
          transpose_items<B / 4>(wu);
          unpack_codes<B, 32>(wu, qp);
        } else if constexpr (B == 6) {
          // a half of a unit is 3 whole words (16 codes): the rows two apart
          // trade packed halves, each half is unpacked on its own, then the
          // adjacent rows trade unpacked quarters
#pragma unroll
          for (int d = 0; d < 3; ++d) {
            const auto a = __builtin_amdgcn_permlane32_swap(wu[d], wu[3 + d], false, false);
            wu[d] = a[0];
            wu[3 + d] = a[1];
          }
          unpack_codes<6, 16>(wu, qp);
          unpack_codes<6, 16>(wu + 3, qp + 8);
          transpose_items<4, false>(qp);
        } else {
          unpack_codes<B, 32>(wu, qp);
          transpose_rows(qp);
        }
        f32x4_t d[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4 bq;
          bq.x = qp[4 * u];
          bq.y = qp[4 * u + 1];
          bq.z = qp[4 * u + 2];
          bq.w = qp[4 * u + 3];
          d[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, aw[u]),
                                                         __builtin_bit_cast(bf16x8_t, bq),
                                                         f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
        }
        // lane = (column j, window rows 4qd + i): units 0..3 in order
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < NACC; ++i) acc[i] = __builtin_fmaf(sv[u], d[u][i], acc[i]);
        continue;
      }
      // A operand and unit sums of every 4-row block (rows past the window
      // read zeros and are never stored); windows of more than 8 rows read
      // each step's operands just before its products, which keeps 48 fewer
      // registers live
      constexpr bool LATE_A = NMB > 2;
      u32x4 av[NMB][4];
      if constexpr (!LATE_A) {
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
          for (int sidx = 0; sidx < 4; ++sidx)
            av[mb][sidx] = *reinterpret_cast<const u32x4*>(smem + a_grp[mb] + r * 64 + sidx * 16);
      }
      // B operand: this lane's unit as 16 exact bf16 pairs
      uint32_t qp[16];
      unpack_codes<B, 32>(wu, qp);
      f32x4_t d[NMB];
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) d[mb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int sidx = 0; sidx < 4; ++sidx) {
        u32x4 bq;
        bq.x = qp[4 * sidx];
        bq.y = qp[4 * sidx + 1];
        bq.z = qp[4 * sidx + 2];
        bq.w = qp[4 * sidx + 3];
        if constexpr (LATE_A) {
#pragma unroll
          for (int mb = 0; mb < NMB; ++mb)
            av[mb][sidx] = *reinterpret_cast<const u32x4*>(smem + a_grp[mb] + r * 64 + sidx * 16);
        }
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb)
          d[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[mb][sidx]),
                                                          __builtin_bit_cast(bf16x8_t, bq), d[mb], 0, 0, 0);
      }
      // lane = (window row 4mb + qd, column j): units q2 = 0..3 in order
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) acc[mb] = __builtin_fmaf(sv[q2], d[mb][q2], acc[mb]);
    }
    if (gr == gr0 + gpp - 1) {
      const int col = (DYN ? c.tile * 16 : (c.tile * ncg + cg) * cw) + j;
      float out[NACC];
      bool store = true;
      if (S == 1) {
#pragma unroll
        for (int mb = 0; mb < NACC; ++mb) out[mb] = acc[mb];
      } else {
        // the column group's parts meet in LDS and are added in part order
#pragma unroll
        for (int mb = 0; mb < NACC; ++mb) reinterpret_cast<float*>(slot)[mb * kWave + lane] = acc[mb];
        __syncthreads();
        store = ks == 0;
        if (store) {
#pragma unroll
          for (int mb = 0; mb < NACC; ++mb) {
            float v = reinterpret_cast<const float*>(slots + static_cast<size_t>(cg * S) * MG::SLOT)[mb * kWave + lane];
            for (int q = 1; q < S; ++q)
              v += reinterpret_cast<const float*>(slots + static_cast<size_t>(cg * S + q) * MG::SLOT)[mb * kWave + lane];
            out[mb] = v;
          }
        }
        __syncthreads();
      }
      if (gu) {
        // lane j + 8 (up) hands its value to lane j (gate) in each 16-lane row
#pragma unroll
        for (int mb = 0; mb < NACC; ++mb) {
          const float u = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(out[mb]), 0x128, 0xf, 0xf, false));
          out[mb] = silu_f32(out[mb]) * u;
        }
      }
      if (store) {
        // (the output's descriptor is built where it is used: its arguments
        // are not needed before the first loads)
        const __amdgpu_buffer_rsrc_t yres = make_rsrc(p.y, p.y_bytes);
#pragma unroll
        for (int mb = 0; mb < NACC; ++mb) {
          const int em = WIDE ? 4 * qd + mb : 4 * mb + qd;
          const bool ok = em < mcount && col < n && j < cw;
          const int off = ok ? static_cast<int>((s_yoff[ok ? em : 0] + mapped_column(p, col)) * 4) : kNoOffset;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gu ? out[mb] : apply_epi(out[mb], p.epi)), yres,
                                                off, 0, 0);
        }
      }
      acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  // a stage's groups one after the other, in order
  auto compute = [&](const Stage& sg, const Cursor& c) {
#pragma unroll
    for (int g2 = 0; g2 < NG; ++g2)
      compute_group(sg.w[g2], sg.s[g2], sg.b[g2], sg.cs + g2 * (CW / 2), sg.cb + g2 * (CW / 2), c, c.gr + g2);
  };

  // A pass's first loads: each thread's first staging item, then the first
  // group's weights.  A wave's loads complete in issue order, so the staging
  // waits for its activations only, not for the weights behind them.  Every
  // thread loads (one past the pass's staging items reads the pass's first
  // unit, which always exists, and never uses it): with no branch ahead of
  // them, only address arithmetic precedes a block's first loads.
  uint32_t xfirst[16];
  Stage sa, sb;
  Cursor cl, cc;
  auto issue_pass = [&](int c0) {
    const int nst = min(MB, total - c0) * units;
    int mi, un;
    split_units(tid < nst ? tid : 0, units, inv_units, mi, un);
    const int e = c0 + mi;
    const int row = IDX ? s_list[e] / p.slots : e;
    const u32x4* src = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(row) * p.k +
                                                      static_cast<int64_t>(un) * 32);
#pragma unroll
    for (int pc = 0; pc < 4; ++pc) {
      const u32x4 v = src[pc];
      xfirst[4 * pc] = v.x;
      xfirst[4 * pc + 1] = v.y;
      xfirst[4 * pc + 2] = v.z;
      xfirst[4 * pc + 3] = v.w;
    }
    // (keeps the activations' loads ahead of the weights' in issue order)
    asm volatile("" ::: "memory");
    cl = Cursor{DYN ? u0 + wv : bx, gr0, 0};
    load_stage(sa, cl);
    // (and the weights' loads ahead of the pass's LDS work)
    asm volatile("" ::: "memory");
    advance(cl);
  };
  auto set_p_off = [&]() {
#pragma unroll
    for (int t = 0; t < NP; ++t) {
      const int pc = qd * NP + t, ln = pc / 8, pp = pc % 8;
      p_off[t] = ((ln * 16 + j) * 8 + ((pp + j / 2) & 7)) * 16;
    }
  };
  for (int c0 = 0; c0 < total; c0 += MB) {
    issue_pass(c0);
    mcount = min(MB, total - c0);
    const int nstage = mcount * units;
    cc = Cursor{bx, gr0, 0};
    if (tid < mcount) {
      const int e = c0 + tid;
      if (IDX) {
        const int t = s_list[e];
        const int row = t / p.slots, sl = t % p.slots;
        s_xrow[tid] = row;
        s_yoff[tid] = (static_cast<int64_t>(row) * p.slots + sl) * p.n;
      } else {
        s_xrow[tid] = e;
        s_yoff[tid] = static_cast<int64_t>(e) * p.ldy;
      }
    }
    if (DYN && tid == 0) *s_next = u0 + 2 * NW;   // read after the barrier below
    for (int t = tid; t < ZB / 4; t += NT) reinterpret_cast<uint32_t*>(zero_area)[t] = 0u;
    set_bases();
    __syncthreads();
    // ---- stage the window: each unit's activations in slot order, and its sum ----
    for (int t = tid; t < nstage; t += NT) {
      int mi, un;
      split_units(t, units, inv_units, mi, un);
      uint32_t xin[16];
      if (t == tid) {
#pragma unroll
        for (int q = 0; q < 16; ++q) xin[q] = xfirst[q];
      } else {
        const u32x4* src = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(s_xrow[mi]) * p.k +
                                                          static_cast<int64_t>(un) * 32);
#pragma unroll
        for (int pc = 0; pc < 4; ++pc) {
          const u32x4 v = src[pc];
          xin[4 * pc] = v.x;
          xin[4 * pc + 1] = v.y;
          xin[4 * pc + 2] = v.z;
          xin[4 * pc + 3] = v.w;
        }
      }
      float X = 0.0f;
      const uint32_t ones = 0x3f803f80u;  // bf16 pair {1, 1}
      u32x4* dst = reinterpret_cast<u32x4*>(smem + mi * xstride + un * 64);
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        u32x4 o;
        o.x = slot_pair<B>(xin, 4 * pc);
        o.y = slot_pair<B>(xin, 4 * pc + 1);
        o.z = slot_pair<B>(xin, 4 * pc + 2);
        o.w = slot_pair<B>(xin, 4 * pc + 3);
        X = dot2(o.x, ones, X);
        X = dot2(o.y, ones, X);
        X = dot2(o.z, ones, X);
        X = dot2(o.w, ones, X);
        dst[pc] = o;
      }
      xsum[mi * sstride + un] = X;
    }
    __syncthreads();
    set_p_off();
    // double-buffered: a group's loads are in flight while the previous one
    // is computed
    if constexpr (DYN) {
      // the compute side follows the stages' own cursors (the units the
      // load side was handed)
      while (sa.cur.tile < tend) {
        load_stage(sb, cl);
        advance(cl);
        compute(sa, sa.cur);
        if (sb.cur.tile >= tend) break;
        load_stage(sa, cl);
        advance(cl);
        compute(sb, sb.cur);
      }
    } else {
      while (cc.tile < tiles) {
        load_stage(sb, cl);
        advance(cl);
        compute(sa, cc);
        advance(cc);
        if (cc.tile >= tiles) break;
        load_stage(sa, cl);
        advance(cl);
        compute(sb, cc);
        advance(cc);
      }
    }
    __syncthreads();    // LDS window reused by the next pass of routed rows
  }
}

// The matrix-core kernels: the block-diagonal and wide forms, plain or
// gate/up pairs, plain/strided or indexed calls.  Pairing and routing are
// compiled in or out, so no kernel holds the registers of a path it never
// takes.  Indexed calls stage at most kIndexedWindow routed rows a pass.
// Waves per SIMD the register allocation must leave room for.  The
// block-diagonal indexed kernels of the routed window (4 rows) with 8-bit
// codes, or 4-bit codes in groups of 64 or 128, fit 96 VGPRs with no spill,
// so a CU holds 5 of their blocks instead of 4: the 4/64 experts (128 x 1024
// x 2048, 16 rows x 8 slots, 1,360 routed blocks) measured 23.9 against
// 24.7 us and the gate/up pair 43.3 against 45.6 us on one box.  (Other
// widths and groups spill at 96.)  Elsewhere the allocator's choice stands.
template <int B, int G, int MB, bool WIDE, bool IDX> struct MinWaves {
  static constexpr int v = (IDX && !WIDE && MB == 4 && (B == 8 || (B == 4 && G >= 64))) ? 5 : 1;
};

#define QG_MFMA_KERNEL(NAME, WIDE, GU, IDX)                                                  \
  template <int B, int G, int MB>                                                            \
  __global__ __launch_bounds__(MWaves<MB>::v * kWave)                                        \
  __attribute__((amdgpu_waves_per_eu(MinWaves<B, G, MB, WIDE, IDX>::v))) void NAME(const Params p) { \
    extern __shared__ __align__(16) unsigned char smem[];                                    \
    __shared__ int s_wave_cnt[MWaves<MB>::v];                                                \
    __shared__ int s_xrow[QGEMV_MAX_WINDOW];                                                 \
    __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];                                             \
    mfma_body<B, G, MB, WIDE, GU, IDX>(p, blockIdx.x, gridDim.x, smem, s_wave_cnt, s_xrow, s_yoff); \
  }
QG_MFMA_KERNEL(qrow_mfma, false, false, false)
QG_MFMA_KERNEL(qrow_mfma_wide, true, false, false)
QG_MFMA_KERNEL(qrow_mfma_gateup, false, true, false)
QG_MFMA_KERNEL(qrow_mfma_wide_gateup, true, true, false)
QG_MFMA_KERNEL(qrow_mfma_indexed, false, false, true)
QG_MFMA_KERNEL(qrow_mfma_wide_indexed, true, false, true)
QG_MFMA_KERNEL(qrow_mfma_gateup_indexed, false, true, true)
QG_MFMA_KERNEL(qrow_mfma_wide_gateup_indexed, true, true, true)
#undef QG_MFMA_KERNEL

// The tile walk's 8- and 16-row windows in blocks of 4 waves, for plain and
// strided calls on small matrices, whose 8-wave blocks would leave CUs idle
// (two waves a SIMD on half the CUs or fewer): one wave a SIMD on twice the
// CUs, each block staging the window for fewer waves.  A column's arithmetic
// does not depend on its block, so the bits are those of the 8-wave blocks.
#define QG_MFMA4_KERNEL(NAME, WIDE)                                                           \
  template <int B, int G, int MB>                                                            \
  __global__ __launch_bounds__(4 * kWave) void NAME(const Params p) {                       \
    extern __shared__ __align__(16) unsigned char smem[];                                    \
    __shared__ int s_wave_cnt[4];                                                            \
    __shared__ int s_xrow[QGEMV_MAX_WINDOW];                                                 \
    __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];                                             \
    mfma_body<B, G, MB, WIDE, false, false, false, const Params, 4>(p, blockIdx.x, gridDim.x, smem, \
                                                                   s_wave_cnt, s_xrow, s_yoff); \
  }
QG_MFMA4_KERNEL(qrow_mfma_w4, false)
QG_MFMA4_KERNEL(qrow_mfma_wide_w4, true)
#undef QG_MFMA4_KERNEL

// The block-diagonal kernels for matrices of many columns: one block of
// DynWaves waves per CU, its 16-column units handed out in the block.
#define QG_DYN_KERNEL(NAME, WIDE)                                                             \
  template <int B, int G, int MB>                                                            \
  __global__ __launch_bounds__(dyn_waves(B, G, MB, WIDE) * kWave) void NAME(const Params p) { \
    extern __shared__ __align__(16) unsigned char smem[];                                    \
    __shared__ int s_wave_cnt[DynWaves<B, G, MB, WIDE>::v];                                  \
    __shared__ int s_xrow[QGEMV_MAX_WINDOW];                                                 \
    __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];                                             \
    __shared__ int s_next;                                                                   \
    mfma_body<B, G, MB, WIDE, false, false, true>(p, blockIdx.x, gridDim.x, smem, s_wave_cnt, s_xrow, \
                                                  s_yoff, &s_next);                          \
  }
QG_DYN_KERNEL(qrow_mfma_dyn, false)
QG_DYN_KERNEL(qrow_mfma_wide_dyn, true)
#undef QG_DYN_KERNEL

// ---------------------------------------------------------------------------
// Fused stack: the runs of a fused projection (each a matrix of one width and
// group whose members write their own output columns) in one dispatch.  The
// blocks are split among the runs; each run executes exactly the body of its
// own strided call, so every member's bits equal that call's.
// ---------------------------------------------------------------------------

// A run's body and block count side by side: one 8-byte argument read
// gives a block both.
struct RunSel {
  int32_t kind;       // which body: see the two kernels below
  int32_t nblocks;    // blocks of the run
};

struct StackParams {
  Params run[kMaxRuns];
  RunSel sel[kMaxRuns];
  int32_t nruns;
};

// A fused stack's run read in place in the kernel's argument segment
// (address space 4): loads through it are scalar loads at a uniform offset,
// which the compiler issues where a field is used and may issue again
// instead of holding the value, exactly as for a kernel's own by-value
// Params.  (A Params copy selected at run time holds every field in scalar
// registers from the start of the body; indexing the by-value StackParams
// at run time copies all of it to scratch.)
typedef const __attribute__((address_space(4))) Params KParams;
typedef const __attribute__((address_space(4))) uint64_t KSel;

// The block's run is blockIdx.y (one grid row per run), its place among
// that run's blocks blockIdx.x; a row's blocks past its run's block count
// leave at once.  StackParams is the kernel's only argument, so it starts
// the argument segment.
#define QG_SELECT_RUN(p, bx, gx, kind)                                                          \
  const char __attribute__((address_space(4)))* args_ =                                         \
      (const char __attribute__((address_space(4)))*)(__builtin_amdgcn_kernarg_segment_ptr());  \
  const int r_ = static_cast<int>(blockIdx.y);                                                  \
  KParams& p = reinterpret_cast<KParams*>(args_ + offsetof(StackParams, run))[r_];              \
  const uint64_t sel_ = reinterpret_cast<KSel*>(args_ + offsetof(StackParams, sel))[r_];        \
  const int gx = static_cast<int>(sel_ >> 32);         /* RunSel::nblocks */                    \
  const int kind = static_cast<int>(sel_ & 0xffffffffu); /* RunSel::kind */                     \
  const int bx = static_cast<int>(blockIdx.x);                                                  \
  if (bx >= gx) return

static_assert(offsetof(StackParams, sel) % 8 == 0 && offsetof(RunSel, kind) == 0 &&
                  offsetof(RunSel, nblocks) == 4 && sizeof(RunSel) == 8,
              "one 8-byte read per run, kind in its low half");

// Dot-form runs: kind = (bits index * 3 + group index) * 2 + staging.
template <int MB>
__global__ __launch_bounds__(kThreads) void qrow_stack(const StackParams sp) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_list[kMaxList];
  __shared__ int s_wave_cnt[kWaves];
  __shared__ int s_xrow[QGEMV_MAX_WINDOW];
  __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];
  (void)sp;
  QG_SELECT_RUN(p, bx, gx, kind);
// (the empty asm keeps each case's parameter loads inside the case, so no
// value is live across the switch)
#define QG_BODY(B, G, STG)               \
  do {                                   \
    asm volatile("" ::: "memory");       \
    fast_body<B, G, MB, STG>(p, bx, gx, smem, s_list, s_wave_cnt, s_xrow, s_yoff); \
  } while (0)
#define QG_PAIR(BI, B, GI, G)                  \
  case ((BI) * 3 + (GI)) * 2:                   \
    QG_BODY(B, G, false);                       \
    break;                                      \
  case ((BI) * 3 + (GI)) * 2 + 1:               \
    if constexpr (Geo<B>::PPC > 1) QG_BODY(B, G, true); \
    break;
#define QG_WIDTH(BI, B) QG_PAIR(BI, B, 0, 32) QG_PAIR(BI, B, 1, 64) QG_PAIR(BI, B, 2, 128)
  switch (kind) {
    QG_WIDTH(0, 2)
    QG_WIDTH(1, 3)
    QG_WIDTH(2, 4)
    QG_WIDTH(3, 5)
    QG_WIDTH(4, 6)
    QG_WIDTH(5, 8)
    default:
      break;
  }
#undef QG_WIDTH
#undef QG_PAIR
#undef QG_BODY
}

// Matrix-core runs: kind = bits index * 3 + group index.  16-row windows
// take the wide bodies (the same bits as the block-diagonal ones).
template <int MB>
__global__ __launch_bounds__(MWaves<MB>::v * kWave) void qrow_stack_mfma(const StackParams sp) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int s_wave_cnt[MWaves<MB>::v];
  __shared__ int s_xrow[QGEMV_MAX_WINDOW];
  __shared__ int64_t s_yoff[QGEMV_MAX_WINDOW];
  (void)sp;
  QG_SELECT_RUN(p, bx, gx, kind);
#define QG_BODY(B, G)                    \
  do {                                   \
    asm volatile("" ::: "memory");       \
    mfma_body<B, G, MB, (MB >= 16)>(p, bx, gx, smem, s_wave_cnt, s_xrow, s_yoff); \
  } while (0)
#define QG_PAIR(BI, B, GI, G) \
  case (BI) * 3 + (GI):       \
    QG_BODY(B, G);            \
    break;
#define QG_WIDTH(BI, B) QG_PAIR(BI, B, 0, 32) QG_PAIR(BI, B, 1, 64) QG_PAIR(BI, B, 2, 128)
  switch (kind) {
    QG_WIDTH(0, 2)
    QG_WIDTH(1, 3)
    QG_WIDTH(2, 4)
    QG_WIDTH(3, 5)
    QG_WIDTH(4, 6)
    QG_WIDTH(5, 8)
    default:
      break;
  }
#undef QG_WIDTH
#undef QG_PAIR
#undef QG_BODY
}

// The product kernels' own unpack, written back as integer codes.
template <int B>
__global__ __launch_bounds__(kThreads) void unpack_kernel(const uint32_t* __restrict__ w, int64_t n,
                                                          int64_t k, uint8_t* __restrict__ codes) {
  const int64_t units = k / 32;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= n * units) return;
  const int64_t row = t / units, u = t % units;
  uint32_t wu[B];
  const uint32_t* src = w + row * (k * B / 32) + u * B;
#pragma unroll
  for (int i = 0; i < B; ++i) wu[i] = src[i];
  uint32_t q[16];
  unpack_codes<B, 32>(wu, q);
  uint8_t* dst = codes + row * k + u * 32;
#pragma unroll
  for (int pp = 0; pp < 16; ++pp) {
    dst[slot_code<B>(2 * pp)] = static_cast<uint8_t>(__uint_as_float(q[pp] << 16));
    dst[slot_code<B>(2 * pp + 1)] = static_cast<uint8_t>(__uint_as_float(q[pp] & 0xffff0000u));
  }
}

// ---------------------------------------------------------------------------
// kernel table
// ---------------------------------------------------------------------------

typedef void (*KernelFn)(const Params);

constexpr int kBits[6] = {2, 3, 4, 5, 6, 8};
constexpr int kGroups[3] = {32, 64, 128};
constexpr int kWindows[5] = {1, 2, 4, 8, 16};
constexpr int kIndexedWindow = 4;  // routed rows staged per pass
static_assert(kIndexedWindow == 4, "indexed matrix-core kernels exist for 1, 2 and 4 rows");

struct Entry {
  KernelFn fast[5][2];  // by window variant and staging (0: direct loads, 1: LDS hand-off)
  KernelFn generic[5];  // by window variant: one-unit chunks, any lane count
  int fast_rows[5];     // columns per lane of the fast kernels
  int generic_rows[5];
  KernelFn mfma[5];     // matrix-core kernels by window variant
  KernelFn mfma_gateup[5];  // the same for gate/up pairs
  KernelFn mfma_indexed[3];         // indexed calls (windows of 1, 2 and 4 routed rows)
  KernelFn mfma_gateup_indexed[3];  // indexed gate/up pairs
  KernelFn mfma_dyn[5];  // units handed out in the block, by window variant (null: not built)
  KernelFn mfma4[2];     // the 8- and 16-row variants in 4-wave blocks (small matrices)
  int mfma_slot;        // bytes of one wave's LDS slot (one load group)
  int mfma_waves[5];    // waves per block of the matrix-core kernels by window variant
  int mfma_group;       // 128-code rounds per load group (k is a multiple of 128 * this)
  int mfma_salign;      // alignment the scale and bias arrays need (bytes)
  int dyn_stage;        // load groups per stage of the kernels that hand out units (k: 128 * group * this)
  int dyn_salign;       // the scale and bias alignment those kernels need (their combined scale loads)
};

template <int B, int G>
Entry make_entry() {
  Entry e{};
  e.fast[0][0] = qrow_fast<B, G, 1, false>;
  e.fast[1][0] = qrow_fast<B, G, 2, false>;
  e.fast[2][0] = qrow_fast<B, G, 4, false>;
  e.fast[3][0] = qrow_fast<B, G, 8, false>;
  e.fast[4][0] = qrow_fast<B, G, 16, false>;
  if constexpr (Geo<B>::PPC > 1) {
    e.fast[0][1] = qrow_fast<B, G, 1, true>;
    e.fast[1][1] = qrow_fast<B, G, 2, true>;
    e.fast[2][1] = qrow_fast<B, G, 4, true>;
    e.fast[3][1] = qrow_fast<B, G, 8, true>;
    e.fast[4][1] = qrow_fast<B, G, 16, true>;
  }
  e.generic[0] = qrow_generic<B, G, 1, 1>;
  e.generic[1] = qrow_generic<B, G, 1, 2>;
  e.generic[2] = qrow_generic<B, G, 1, 4>;
  e.generic[3] = qrow_generic<B, G, 1, 8>;
  e.generic[4] = qrow_generic<B, G, 1, 16>;
  e.fast_rows[0] = FastRows<B, 1>::v;
  e.fast_rows[1] = FastRows<B, 2>::v;
  e.fast_rows[2] = FastRows<B, 4>::v;
  e.fast_rows[3] = FastRows<B, 8>::v;
  e.fast_rows[4] = FastRows<B, 16>::v;
  e.generic_rows[0] = RowsPerLane<B, 1>::v;
  e.generic_rows[1] = RowsPerLane<B, 2>::v;
  e.generic_rows[2] = RowsPerLane<B, 4>::v;
  e.generic_rows[3] = RowsPerLane<B, 8>::v;
  e.generic_rows[4] = RowsPerLane<B, 16>::v;
  e.mfma_dyn[0] = qrow_mfma_dyn<B, G, 1>;
  e.mfma_dyn[1] = qrow_mfma_dyn<B, G, 2>;
  e.mfma_dyn[2] = qrow_mfma_dyn<B, G, 4>;
  e.mfma_dyn[3] = qrow_mfma_dyn<B, G, 8>;
  e.mfma_dyn[4] = qrow_mfma_dyn<B, G, 16>;
  e.mfma[0] = qrow_mfma<B, G, 1>;
  e.mfma[1] = qrow_mfma<B, G, 2>;
  e.mfma[2] = qrow_mfma<B, G, 4>;
  e.mfma[3] = qrow_mfma<B, G, 8>;
  e.mfma[4] = qrow_mfma<B, G, 16>;
  e.mfma4[0] = qrow_mfma_w4<B, G, 8>;
  e.mfma4[1] = qrow_mfma_w4<B, G, 16>;
  e.mfma_gateup[0] = qrow_mfma_gateup<B, G, 1>;
  e.mfma_gateup[1] = qrow_mfma_gateup<B, G, 2>;
  e.mfma_gateup[2] = qrow_mfma_gateup<B, G, 4>;
  e.mfma_gateup[3] = qrow_mfma_gateup<B, G, 8>;
  e.mfma_gateup[4] = qrow_mfma_gateup<B, G, 16>;
  e.mfma_indexed[0] = qrow_mfma_indexed<B, G, 1>;
  e.mfma_indexed[1] = qrow_mfma_indexed<B, G, 2>;
  e.mfma_indexed[2] = qrow_mfma_indexed<B, G, 4>;
  e.mfma_gateup_indexed[0] = qrow_mfma_gateup_indexed<B, G, 1>;
  e.mfma_gateup_indexed[1] = qrow_mfma_gateup_indexed<B, G, 2>;
  e.mfma_gateup_indexed[2] = qrow_mfma_gateup_indexed<B, G, 4>;
  e.mfma_slot = MGroup<B, G>::SLOT;
  e.mfma_group = MGroup<B, G>::R;
  e.mfma_waves[0] = MWaves<1>::v;
  e.mfma_waves[1] = MWaves<2>::v;
  e.mfma_waves[2] = MWaves<4>::v;
  e.mfma_waves[3] = MWaves<8>::v;
  e.mfma_waves[4] = MWaves<16>::v;
  e.mfma_salign = MGroup<B, G>::S16 ? 16 : 4;
  e.dyn_stage = dyn_stage_groups(B);
  using MG = MGroup<B, G>;
  e.dyn_salign = (dyn_stage_groups(B) == 2 && !MG::S16 && MG::SB >= 4) ? 2 * MG::SB : e.mfma_salign;
  return e;
}

// The wide-window matrix-core kernels of one (bits, group) by window variant.
struct WideEntry {
  KernelFn k[5];
  KernelFn k4[2];       // the 8- and 16-row variants in 4-wave blocks (small matrices)
  KernelFn dyn[5];      // units handed out in the block (null: not built)
  KernelFn gateup[5];   // gate/up pairs
  KernelFn indexed[3];  // indexed calls (windows of 1, 2 and 4 routed rows)
  KernelFn gateup_indexed[3];
};

template <int B, int G>
WideEntry make_wide_entry() {
  WideEntry e{};
  e.dyn[0] = qrow_mfma_wide_dyn<B, G, 1>;
  e.dyn[1] = qrow_mfma_wide_dyn<B, G, 2>;
  e.dyn[2] = qrow_mfma_wide_dyn<B, G, 4>;
  e.dyn[3] = qrow_mfma_wide_dyn<B, G, 8>;
  e.dyn[4] = qrow_mfma_wide_dyn<B, G, 16>;
  e.k[0] = qrow_mfma_wide<B, G, 1>;
  e.k[1] = qrow_mfma_wide<B, G, 2>;
  e.k[2] = qrow_mfma_wide<B, G, 4>;
  e.k[3] = qrow_mfma_wide<B, G, 8>;
  e.k[4] = qrow_mfma_wide<B, G, 16>;
  e.k4[0] = qrow_mfma_wide_w4<B, G, 8>;
  e.k4[1] = qrow_mfma_wide_w4<B, G, 16>;
  e.gateup[0] = qrow_mfma_wide_gateup<B, G, 1>;
  e.gateup[1] = qrow_mfma_wide_gateup<B, G, 2>;
  e.gateup[2] = qrow_mfma_wide_gateup<B, G, 4>;
  e.gateup[3] = qrow_mfma_wide_gateup<B, G, 8>;
  e.gateup[4] = qrow_mfma_wide_gateup<B, G, 16>;
  e.indexed[0] = qrow_mfma_wide_indexed<B, G, 1>;
  e.indexed[1] = qrow_mfma_wide_indexed<B, G, 2>;
  e.indexed[2] = qrow_mfma_wide_indexed<B, G, 4>;
  e.gateup_indexed[0] = qrow_mfma_wide_gateup_indexed<B, G, 1>;
  e.gateup_indexed[1] = qrow_mfma_wide_gateup_indexed<B, G, 2>;
  e.gateup_indexed[2] = qrow_mfma_wide_gateup_indexed<B, G, 4>;
  return e;
}

// One table of kernels per code width, each built in its own translation
// unit: index [group 32/64/128].
const Entry* entries_b2();
const Entry* entries_b3();
const Entry* entries_b4();
const Entry* entries_b5();
const Entry* entries_b6();
const Entry* entries_b8();
const WideEntry* wide_entries_b2();
const WideEntry* wide_entries_b3();
const WideEntry* wide_entries_b4();
const WideEntry* wide_entries_b5();
const WideEntry* wide_entries_b6();
const WideEntry* wide_entries_b8();

// Fused-stack kernels (both arithmetic forms) by window variant (1, 2, 4,
// 8, 16 rows), one translation unit each.
typedef void (*StackFn)(const StackParams);
struct StackKernels {
  StackFn dot;    // qrow_stack<MB>
  StackFn mfma;   // qrow_stack_mfma<MB>
};
StackKernels stack_kernels_m1();
StackKernels stack_kernels_m2();
StackKernels stack_kernels_m4();
StackKernels stack_kernels_m8();
StackKernels stack_kernels_m16();

}  // namespace qg
