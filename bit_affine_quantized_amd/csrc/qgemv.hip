// qgemv.hip — MLX-affine quantized row product for gfx950 (MI355X).
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
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "qgemv.h"

namespace qg {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxSlots = 64;
constexpr int kMaxList = QGEMV_MAX_WINDOW * kMaxSlots;
// 160 KiB of LDS per CU on gfx950, less the kernels' static arrays.
constexpr size_t kMaxDynamicLds = 160 * 1024 - 8 * 1024;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 32-code units per lane chunk: the smallest whole number of units that is
// also a whole number of 16-byte loads.
template <int B> struct Units;
template <> struct Units<2> { static constexpr int v = 2; };
template <> struct Units<3> { static constexpr int v = 4; };
template <> struct Units<4> { static constexpr int v = 1; };
template <> struct Units<5> { static constexpr int v = 4; };
template <> struct Units<6> { static constexpr int v = 2; };
template <> struct Units<8> { static constexpr int v = 1; };

// Output columns each lane carries side by side (more loads in flight,
// activations read from LDS once for all of them).
template <int B, int MB> struct RowsPerLane {
  static constexpr int v = (MB == 1) ? ((B == 2 || B == 4 || B == 8) ? 4 : 2) : 2;
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

template <int B, int P>
__device__ __forceinline__ void unpack_pairs_generic(const uint32_t* w, uint32_t* q) {
  if constexpr (P < 16) {
    q[P] = pack_bf16x2(static_cast<float>(unit_code<B, 2 * P>(w)),
                       static_cast<float>(unit_code<B, 2 * P + 1>(w)));
    unpack_pairs_generic<B, P + 1>(w, q);
  }
}

// One 32-code unit (B words) -> 16 bf16 pairs q[p] = {code 2p, code 2p+1}.
template <int B>
__device__ __forceinline__ void unpack_unit(const uint32_t* w, uint32_t* q) {
  if constexpr (B == 8) {
#pragma unroll
    for (int wi = 0; wi < 8; ++wi) {
      const uint32_t v = w[wi];
      q[2 * wi] = pack_bf16x2(static_cast<float>(v & 0xffu), static_cast<float>((v >> 8) & 0xffu));
      q[2 * wi + 1] = pack_bf16x2(static_cast<float>((v >> 16) & 0xffu), static_cast<float>(v >> 24));
    }
  } else if constexpr (B == 4) {
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      const uint32_t lo = w[wi] & 0x0f0f0f0fu;          // codes 0,2,4,6 of the word
      const uint32_t hi = (w[wi] >> 4) & 0x0f0f0f0fu;   // codes 1,3,5,7
#pragma unroll
      for (int b = 0; b < 4; ++b)
        q[4 * wi + b] = pack_bf16x2(static_cast<float>((lo >> (8 * b)) & 0xffu),
                                    static_cast<float>((hi >> (8 * b)) & 0xffu));
    }
  } else if constexpr (B == 2) {
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
      uint32_t t[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) t[s] = (w[wi] >> (2 * s)) & 0x03030303u;  // code 4b+s in byte b
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        q[8 * wi + 2 * b] = pack_bf16x2(static_cast<float>((t[0] >> (8 * b)) & 0xffu),
                                        static_cast<float>((t[1] >> (8 * b)) & 0xffu));
        q[8 * wi + 2 * b + 1] = pack_bf16x2(static_cast<float>((t[2] >> (8 * b)) & 0xffu),
                                            static_cast<float>((t[3] >> (8 * b)) & 0xffu));
      }
    }
  } else {
    unpack_pairs_generic<B, 0>(w, q);
  }
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
  const uint32_t* w;        // [E][N][WPR]
  const uint16_t* scales;   // [E][N][GPR]
  const uint16_t* biases;
  const uint16_t* x;        // [M][K] bf16
  float* y;
  const int32_t* idx;       // indexed: [M][slots]
  int64_t n;                // output columns
  int64_t k;
  int64_t wpr;              // words per row
  int64_t gpr;              // groups per row
  int64_t ldy;              // plain/strided row stride of y
  int32_t m;                // window rows
  int32_t slots;            // indexed only
  int32_t n_experts;
  int32_t epi;
  int32_t lpr;              // lanes per output column (power of two <= 64)
  int32_t cpl;              // chunks per lane
  int32_t nchunks;          // chunks per row = lpr * cpl
  int32_t tiles;            // column tiles per expert
  int32_t indexed;          // 0: plain/strided, 1: indexed
};

__device__ __forceinline__ float apply_epi(float v, int epi) {
  if (epi == QGEMV_EPI_RELU2) return v > 0.0f ? v * v : (v != v ? v : 0.0f);
  return v;
}

// Block-wide list of the (row, slot) pairs routed to `expert`, in index
// order.  Returns the count.
__device__ int build_route_list(const int32_t* __restrict__ idx, int total, int expert,
                                int* list, int* wave_cnt) {
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  int base_count = 0;
  for (int base = 0; base < total; base += kThreads) {
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
    for (int i = 0; i < kWaves; ++i) all += wave_cnt[i];
    __syncthreads();
    base_count += all;
  }
  return base_count;
}

template <int B, int G, int UPC, int MB>
__global__ __launch_bounds__(kThreads) void qrow_kernel(const Params p) {
  constexpr int WPC = B * UPC;              // words per lane chunk
  constexpr int UPG = G / 32;               // units per group
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

  for (int c0 = 0; c0 < total; c0 += MB) {
    const int mcount = min(MB, total - c0);
    // ---- stage the window: x pieces and per-unit activation sums ----
    if (tid < MB) {
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
    }
    __syncthreads();
    for (int t = tid; t < mcount * units; t += kThreads) {
      const int mi = t / units, u = t % units;
      const int c = u / UPC, ui = u % UPC;
      const u32x4* src = reinterpret_cast<const u32x4*>(p.x + static_cast<int64_t>(s_xrow[mi]) * p.k +
                                                        static_cast<int64_t>(u) * 32);
      u32x4 v[4];
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) v[pc] = src[pc];
      float X = 0.0f;
      const uint32_t ones = 0x3f803f80u;  // bf16 pair {1, 1}
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) {
        X = dot2(v[pc].x, ones, X);
        X = dot2(v[pc].y, ones, X);
        X = dot2(v[pc].z, ones, X);
        X = dot2(v[pc].w, ones, X);
        xs[((mi * UPC + ui) * 4 + pc) * nchunks + c] = v[pc];
      }
      xsum[(mi * UPC + ui) * nchunks + c] = X;
    }
    __syncthreads();

    // ---- column tiles of this block ----
    for (int tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
      const int64_t col0 = static_cast<int64_t>(tile) * tile_rows + wv * slots_per_wave * R + slot;
      int64_t col[R];
#pragma unroll
      for (int r = 0; r < R; ++r) col[r] = col0 + r * slots_per_wave;

      float acc[R][MB];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) acc[r][mi] = 0.0f;

      for (int j = 0; j < p.cpl; ++j) {
        const int c = li + lpr * j;
        uint32_t wr[R][WPC];
        float sc[R][UPC], bi[R][UPC];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int64_t cr = col[r] < p.n ? col[r] : p.n - 1;
          load_chunk<WPC>(wbase + cr * p.wpr + static_cast<int64_t>(c) * WPC, wr[r]);
#pragma unroll
          for (int ui = 0; ui < UPC; ++ui) {
            const int64_t g = (static_cast<int64_t>(c) * UPC + ui) / UPG;
            sc[r][ui] = bf16_to_f32(sbase[cr * p.gpr + g]);
            bi[r][ui] = bf16_to_f32(bbase[cr * p.gpr + g]);
          }
        }
#pragma unroll
        for (int ui = 0; ui < UPC; ++ui) {
          uint32_t q[R][16];
#pragma unroll
          for (int r = 0; r < R; ++r) unpack_unit<B>(&wr[r][ui * B], q[r]);
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
                acc[r][mi] = __builtin_fmaf(sc[r][ui], a, acc[r][mi]);
                acc[r][mi] = __builtin_fmaf(bi[r][ui], X, acc[r][mi]);
              }
            }
          }
        }
      }

      // ---- reduce over the lpr lanes of each column (fixed xor tree) ----
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
          float v = acc[r][mi];
          for (int off = lpr >> 1; off > 0; off >>= 1) v += __shfl_xor(v, off);
          acc[r][mi] = v;
        }
      if (li == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (col[r] < p.n) {
#pragma unroll
            for (int mi = 0; mi < MB; ++mi)
              if (mi < mcount) p.y[s_yoff[mi] + col[r]] = apply_epi(acc[r][mi], p.epi);
          }
        }
      }
    }
    __syncthreads();  // LDS window reused by the next chunk of routed rows
  }
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
  unpack_unit<B>(wu, q);
  uint8_t* dst = codes + row * k + u * 32;
#pragma unroll
  for (int pp = 0; pp < 16; ++pp) {
    dst[2 * pp] = static_cast<uint8_t>(__uint_as_float(q[pp] << 16));
    dst[2 * pp + 1] = static_cast<uint8_t>(__uint_as_float(q[pp] & 0xffff0000u));
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

struct Entry {
  KernelFn main[5];     // by window variant, chunked geometry
  KernelFn unit[5];     // by window variant, one-unit chunks (fallback)
};

template <int B, int G, int UPC>
constexpr void fill(KernelFn* f) {
  f[0] = qrow_kernel<B, G, UPC, 1>;
  f[1] = qrow_kernel<B, G, UPC, 2>;
  f[2] = qrow_kernel<B, G, UPC, 4>;
  f[3] = qrow_kernel<B, G, UPC, 8>;
  f[4] = qrow_kernel<B, G, UPC, 16>;
}

template <int B, int G>
Entry make_entry() {
  Entry e{};
  fill<B, G, Units<B>::v>(e.main);
  fill<B, G, 1>(e.unit);
  return e;
}

template <int B>
constexpr int units_of() { return Units<B>::v; }

static int bits_index(int bits) {
  for (int i = 0; i < 6; ++i)
    if (kBits[i] == bits) return i;
  return -1;
}
static int group_index(int g) {
  for (int i = 0; i < 3; ++i)
    if (kGroups[i] == g) return i;
  return -1;
}

static const Entry& entry(int bi, int gi) {
#define QG_ROW(B) {make_entry<B, 32>(), make_entry<B, 64>(), make_entry<B, 128>()}
  static const Entry table[6][3] = {QG_ROW(2), QG_ROW(3), QG_ROW(4), QG_ROW(5), QG_ROW(6), QG_ROW(8)};
#undef QG_ROW
  return table[bi][gi];
}

static int units_per_chunk(int bits) {
  switch (bits) {
    case 2: return units_of<2>();
    case 3: return units_of<3>();
    case 4: return units_of<4>();
    case 5: return units_of<5>();
    case 6: return units_of<6>();
    case 8: return units_of<8>();
  }
  return 1;
}

static int rows_per_lane(int bits, int mb) {
  switch (bits) {
    case 2: return mb == 1 ? RowsPerLane<2, 1>::v : RowsPerLane<2, 2>::v;
    case 3: return mb == 1 ? RowsPerLane<3, 1>::v : RowsPerLane<3, 2>::v;
    case 4: return mb == 1 ? RowsPerLane<4, 1>::v : RowsPerLane<4, 2>::v;
    case 5: return mb == 1 ? RowsPerLane<5, 1>::v : RowsPerLane<5, 2>::v;
    case 6: return mb == 1 ? RowsPerLane<6, 1>::v : RowsPerLane<6, 2>::v;
    case 8: return mb == 1 ? RowsPerLane<8, 1>::v : RowsPerLane<8, 2>::v;
  }
  return 1;
}

static KernelFn unpack_fn(int bits) {
  switch (bits) {
    case 2: return reinterpret_cast<KernelFn>(unpack_kernel<2>);
    case 3: return reinterpret_cast<KernelFn>(unpack_kernel<3>);
    case 4: return reinterpret_cast<KernelFn>(unpack_kernel<4>);
    case 5: return reinterpret_cast<KernelFn>(unpack_kernel<5>);
    case 6: return reinterpret_cast<KernelFn>(unpack_kernel<6>);
    case 8: return reinterpret_cast<KernelFn>(unpack_kernel<8>);
  }
  return nullptr;
}

}  // namespace qg

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

struct qgemv_handle {
  qgemv_desc d;
  int upc;               // units per lane chunk of the chosen geometry
  int unit_geometry;     // 1: fallback one-unit chunks
  int lpr, cpl, nchunks;
  int64_t wpr, gpr;
  qg::KernelFn fn[5];
  int rows_per_lane[5];
};

namespace {

// Per-device facts, fetched once per device at the first launch on it:
// the compute-unit count and the kernels' dynamic-LDS limit.
struct DeviceInfo {
  std::once_flag once;
  int cus = 0;
  int status = QGEMV_E_HIP;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];

void init_device(DeviceInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return;
  for (int bi = 0; bi < 6; ++bi)
    for (int gi = 0; gi < 3; ++gi) {
      const qg::Entry& e = qg::entry(bi, gi);
      for (int v = 0; v < 5; ++v)
        for (qg::KernelFn fn : {e.main[v], e.unit[v]})
          if (hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                  static_cast<int>(qg::kMaxDynamicLds)) != hipSuccess)
            return;
    }
  info->cus = cus;
  info->status = QGEMV_OK;
}

// The current device's facts, or nullptr when HIP has no usable device.
const DeviceInfo* current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  DeviceInfo* info = &g_devices[dev];
  std::call_once(info->once, init_device, info);
  return info->status == QGEMV_OK ? info : nullptr;
}

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
  if (!a || !b || !abytes || !bbytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

int window_variant(int m) {
  for (int i = 0; i < 5; ++i)
    if (m <= qg::kWindows[i]) return i;
  return -1;
}

size_t lds_bytes(const qgemv_handle* h, int mb) {
  const size_t units = static_cast<size_t>(h->nchunks) * h->upc;
  return static_cast<size_t>(mb) * units * (64 + 4);
}

int check_y_alias(const qgemv_handle* h, const void* y, size_t ybytes, const void* x, size_t xbytes,
                  const void* idx, size_t idxbytes) {
  const size_t E = static_cast<size_t>(h->d.n_experts);
  const size_t wbytes = E * h->d.n * h->wpr * 4, sbytes = E * h->d.n * h->gpr * 2;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, h->d.w, wbytes) ||
      overlaps(y, ybytes, h->d.scales, sbytes) || overlaps(y, ybytes, h->d.biases, sbytes) ||
      overlaps(y, ybytes, idx, idxbytes))
    return QGEMV_E_ALIAS;
  return QGEMV_OK;
}

int launch(const qgemv_handle* h, const uint16_t* x, int32_t m, float* y, int64_t ldy,
           const int32_t* idx, int32_t slots, int32_t epi, void* stream) {
  const DeviceInfo* dev = current_device();
  if (!dev) return QGEMV_E_HIP;
  const int indexed = idx != nullptr;
  const int var = indexed ? window_variant(qg::kIndexedWindow) : window_variant(m);
  const int mb = qg::kWindows[var];
  if (lds_bytes(h, mb) > qg::kMaxDynamicLds) return QGEMV_E_WINDOW;
  const int R = h->rows_per_lane[var];
  const int slots_per_wave = qg::kWave / h->lpr;
  const int64_t tile_rows = static_cast<int64_t>(qg::kWaves) * slots_per_wave * R;
  const int64_t tiles = (h->d.n + tile_rows - 1) / tile_rows;

  qg::Params p{};
  p.w = h->d.w;
  p.scales = h->d.scales;
  p.biases = h->d.biases;
  p.x = x;
  p.y = y;
  p.idx = idx;
  p.n = h->d.n;
  p.k = h->d.k;
  p.wpr = h->wpr;
  p.gpr = h->gpr;
  p.ldy = ldy;
  p.m = m;
  p.slots = slots;
  p.n_experts = h->d.n_experts;
  p.epi = epi;
  p.lpr = h->lpr;
  p.cpl = h->cpl;
  p.nchunks = h->nchunks;
  p.tiles = static_cast<int32_t>(tiles);
  p.indexed = indexed;

  const size_t lds = lds_bytes(h, mb);
  // Enough blocks to fill every CU several times over, each block walking
  // several tiles so the staged window is reused.
  int64_t blocks = tiles;
  const int64_t cap = static_cast<int64_t>(dev->cus) * 8;
  if (blocks > cap) blocks = cap;
  dim3 grid(static_cast<unsigned>(blocks), indexed ? static_cast<unsigned>(h->d.n_experts) : 1u);
  if (indexed) {
    int64_t per_expert = tiles < 8 ? tiles : 8;
    grid.x = static_cast<unsigned>(per_expert);
  }
  hipLaunchKernelGGL(h->fn[var], grid, dim3(qg::kThreads), lds,
                     static_cast<hipStream_t>(stream), p);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_E_HIP;
}

}  // namespace

extern "C" {

const char* qgemv_strerror(int status) {
  switch (status) {
    case QGEMV_OK: return "QGEMV_OK";
    case QGEMV_E_ARG: return "QGEMV_E_ARG";
    case QGEMV_E_BITS: return "QGEMV_E_BITS";
    case QGEMV_E_GROUP: return "QGEMV_E_GROUP";
    case QGEMV_E_SHAPE: return "QGEMV_E_SHAPE";
    case QGEMV_E_STRIDE: return "QGEMV_E_STRIDE";
    case QGEMV_E_ALIGN: return "QGEMV_E_ALIGN";
    case QGEMV_E_WINDOW: return "QGEMV_E_WINDOW";
    case QGEMV_E_ALIAS: return "QGEMV_E_ALIAS";
    case QGEMV_E_NOKERNEL: return "QGEMV_E_NOKERNEL";
    case QGEMV_E_HIP: return "QGEMV_E_HIP";
  }
  return "QGEMV_E_UNKNOWN";
}

int qgemv_create(const qgemv_desc* d, qgemv_t* out) {
  if (!d || !out) return QGEMV_E_ARG;
  const int bi = qg::bits_index(d->bits);
  if (bi < 0) return QGEMV_E_BITS;
  const int gi = qg::group_index(d->group);
  if (gi < 0) return QGEMV_E_GROUP;
  if (d->n < 1 || d->k < 1 || d->k % d->group != 0 || (d->k * d->bits) % 32 != 0)
    return QGEMV_E_SHAPE;
  if (d->n_experts < 1) return QGEMV_E_SHAPE;
  // index arithmetic in the kernels: columns and tiles in int32, elements in int64
  if (d->n > (int64_t{1} << 30) || d->k > (int64_t{1} << 20) ||
      static_cast<double>(d->n) * d->k * d->n_experts > 1.0e12)
    return QGEMV_E_SHAPE;
  if (!d->w || !d->scales || !d->biases) return QGEMV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(d->w) & 15) || (reinterpret_cast<uintptr_t>(d->scales) & 1) ||
      (reinterpret_cast<uintptr_t>(d->biases) & 1))
    return QGEMV_E_ALIGN;

  qgemv_handle h{};
  h.d = *d;
  h.wpr = d->k * d->bits / 32;
  h.gpr = d->k / d->group;
  // The chunked geometry needs whole chunks per row; otherwise each lane
  // takes one 32-code unit at a time (dword loads for 2/3/5/6 bits).
  int upc = qg::units_per_chunk(d->bits);
  h.unit_geometry = 0;
  if (d->k % (32 * upc) != 0) {
    upc = 1;
    h.unit_geometry = 1;
  }
  h.upc = upc;
  h.nchunks = static_cast<int>(d->k / (32 * upc));
  int lpr = 1;
  while (lpr < 64 && h.nchunks % (lpr * 2) == 0) lpr *= 2;
  h.lpr = lpr;
  h.cpl = h.nchunks / lpr;
  const qg::Entry& e = qg::entry(bi, gi);
  for (int i = 0; i < 5; ++i) {
    h.fn[i] = h.unit_geometry ? e.unit[i] : e.main[i];
    h.rows_per_lane[i] = qg::rows_per_lane(d->bits, qg::kWindows[i]);
    if (!h.fn[i]) return QGEMV_E_NOKERNEL;
  }
  // The one-row window must fit in LDS; wider windows are refused at run
  // time when theirs does not (QGEMV_E_WINDOW).
  if (lds_bytes(&h, 1) > qg::kMaxDynamicLds) return QGEMV_E_SHAPE;

  qgemv_handle* hp = new (std::nothrow) qgemv_handle(h);
  if (!hp) return QGEMV_E_ARG;
  *out = hp;
  return QGEMV_OK;
}

void qgemv_destroy(qgemv_t h) { delete h; }

static int check_run_common(qgemv_t h, const uint16_t* x, int32_t m, const float* y, int32_t epi) {
  if (!h) return QGEMV_E_ARG;
  if (m < 0 || m > QGEMV_MAX_WINDOW) return QGEMV_E_WINDOW;
  if (epi != QGEMV_EPI_NONE && epi != QGEMV_EPI_RELU2) return QGEMV_E_ARG;
  if (m == 0) return QGEMV_OK;
  if (!x || !y) return QGEMV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 3)) return QGEMV_E_ALIGN;
  return QGEMV_OK;
}

int qgemv_run_strided(qgemv_t h, const uint16_t* x, int32_t m, float* y, int64_t ldy, int32_t epi,
                      void* stream) {
  int rc = check_run_common(h, x, m, y, epi);
  if (rc != QGEMV_OK) return rc;
  if (h->d.n_experts != 1) return QGEMV_E_ARG;
  if (ldy < h->d.n) return QGEMV_E_STRIDE;
  if (m == 0) return QGEMV_OK;
  const size_t xbytes = static_cast<size_t>(m) * h->d.k * 2;
  const size_t ybytes = (static_cast<size_t>(m - 1) * ldy + h->d.n) * 4;
  rc = check_y_alias(h, y, ybytes, x, xbytes, nullptr, 0);
  if (rc != QGEMV_OK) return rc;
  return launch(h, x, m, y, ldy, nullptr, 0, epi, stream);
}

int qgemv_run(qgemv_t h, const uint16_t* x, int32_t m, float* y, int32_t epi, void* stream) {
  if (!h) return QGEMV_E_ARG;
  return qgemv_run_strided(h, x, m, y, h->d.n, epi, stream);
}

int qgemv_run_indexed(qgemv_t h, const uint16_t* x, int32_t m, const int32_t* idx, int32_t slots,
                      float* y, int32_t epi, void* stream) {
  int rc = check_run_common(h, x, m, y, epi);
  if (rc != QGEMV_OK) return rc;
  if (slots < 0 || slots > qg::kMaxSlots) return QGEMV_E_ARG;
  if (m == 0 || slots == 0) return QGEMV_OK;
  if (!idx) return QGEMV_E_ARG;
  if (reinterpret_cast<uintptr_t>(idx) & 3) return QGEMV_E_ALIGN;
  const size_t xbytes = static_cast<size_t>(m) * h->d.k * 2;
  const size_t ybytes = static_cast<size_t>(m) * slots * h->d.n * 4;
  rc = check_y_alias(h, y, ybytes, x, xbytes, idx, static_cast<size_t>(m) * slots * 4);
  if (rc != QGEMV_OK) return rc;
  return launch(h, x, m, y, h->d.n, idx, slots, epi, stream);
}

int qgemv_debug_unpack(qgemv_t h, int32_t expert, uint8_t* codes, void* stream) {
  if (!h || !codes) return QGEMV_E_ARG;
  if (expert < 0 || expert >= h->d.n_experts) return QGEMV_E_ARG;
  if (!current_device()) return QGEMV_E_HIP;
  const int64_t n = h->d.n, k = h->d.k;
  const int64_t total = n * (k / 32);
  const int64_t blocks = (total + qg::kThreads - 1) / qg::kThreads;
  const uint32_t* w = h->d.w + static_cast<int64_t>(expert) * n * h->wpr;
  typedef void (*UnpackFn)(const uint32_t*, int64_t, int64_t, uint8_t*);
  UnpackFn fn = reinterpret_cast<UnpackFn>(qg::unpack_fn(h->d.bits));
  if (!fn) return QGEMV_E_NOKERNEL;
  hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(blocks)), dim3(qg::kThreads), 0,
                     static_cast<hipStream_t>(stream), w, n, k, codes);
  return hipGetLastError() == hipSuccess ? QGEMV_OK : QGEMV_E_HIP;
}

int qgemv_query(qgemv_t h, int64_t out[6]) {
  if (!h || !out) return QGEMV_E_ARG;
  const int R = h->rows_per_lane[0];
  out[0] = h->lpr;
  out[1] = (qg::kWave / h->lpr) * R;
  out[2] = 32 * h->upc;
  out[3] = qg::kThreads;
  out[4] = static_cast<int64_t>(qg::kWaves) * (qg::kWave / h->lpr) * R;
  const DeviceInfo* dev = current_device();
  out[5] = dev ? dev->cus : 0;
  return QGEMV_OK;
}

}  // extern "C"
