// qgemv.hip — host side of the C ABI (include/qgemv.h): admission,
// geometry, kernel choice and launches.  The kernels are in
// qgemv_kernels.h, instantiated per width in qgemv_b<bits>.hip.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <mutex>
#include <new>
#include <utility>

#include "qgemv.h"
#include "qgemv_kernels.h"

namespace qg {

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
  static const Entry* const tables[6] = {entries_b2(), entries_b3(), entries_b4(),
                                         entries_b5(), entries_b6(), entries_b8()};
  return tables[bi][gi];
}

static const WideEntry& wide_entry(int bi, int gi) {
  static const WideEntry* const tables[6] = {wide_entries_b2(), wide_entries_b3(), wide_entries_b4(),
                                             wide_entries_b5(), wide_entries_b6(), wide_entries_b8()};
  return tables[bi][gi];
}

// Geometry of the fast kernels per width: 16-byte pieces and codes per chunk.
static void fast_geometry(int bits, int* ppc, int* cpc) {
  switch (bits) {
    case 2: *ppc = Geo<2>::PPC; *cpc = Geo<2>::CPC; return;
    case 3: *ppc = Geo<3>::PPC; *cpc = Geo<3>::CPC; return;
    case 4: *ppc = Geo<4>::PPC; *cpc = Geo<4>::CPC; return;
    case 5: *ppc = Geo<5>::PPC; *cpc = Geo<5>::CPC; return;
    case 6: *ppc = Geo<6>::PPC; *cpc = Geo<6>::CPC; return;
    default: *ppc = Geo<8>::PPC; *cpc = Geo<8>::CPC; return;
  }
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

// Exact widen: unit t of the flattened rows (bin words) is re-cut at bout
// bits per code (bout words), the same integer codes, low code first.
__global__ __launch_bounds__(kThreads) void widen_kernel(const uint32_t* __restrict__ w_in, int bin,
                                                         uint32_t* __restrict__ w_out, int bout,
                                                         int64_t units) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= units) return;
  const uint32_t* src = w_in + t * bin;
  uint32_t* dst = w_out + t * bout;
  const uint32_t mask = (1u << bin) - 1u;
  uint64_t acc = 0;
  int have = 0, wo = 0;
  for (int j = 0; j < 32; ++j) {
    const int bit = j * bin, wi = bit >> 5, sh = bit & 31;
    const uint64_t win = static_cast<uint64_t>(src[wi]) | (wi + 1 < bin ? static_cast<uint64_t>(src[wi + 1]) << 32 : 0);
    acc |= static_cast<uint64_t>(static_cast<uint32_t>(win >> sh) & mask) << have;
    have += bout;
    if (have >= 32) {
      dst[wo++] = static_cast<uint32_t>(acc);
      acc >>= 32;
      have -= 32;
    }
  }
}

// Exact regroup: each group's value repeated for the `ratio` smaller groups
// it splits into (rows stay aligned: a row of g groups becomes g * ratio).
__global__ __launch_bounds__(kThreads) void regroup_kernel(const uint16_t* __restrict__ in,
                                                           uint16_t* __restrict__ out, int ratio,
                                                           int64_t total) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (t < total) out[t] = in[t / ratio];
}

}  // namespace qg

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

struct qgemv_handle {
  qgemv_desc d;
  int fast;              // 1: whole-piece chunks (qrow_fast); 0: one-unit chunks (qrow_generic)
  int ppc, cpc;          // 16-byte pieces and codes per lane chunk
  int lpr, cpl, nchunks; // lanes per column, chunks per lane, chunks per row
  int vec_groups;        // scales/biases aligned for packed loads
  int64_t wpr, gpr;
  int arith;             // QGEMV_ARITH_DOT, QGEMV_ARITH_MFMA or QGEMV_ARITH_WIDE
  int ksplit;            // matrix-core forms: K-parts per column (1, 2 or 4)
  int wide_windows;      // AUTO on the matrix cores: windows of 9-16 rows run the wide kernels
  const qg::Entry* entry;
  const qg::WideEntry* wide;
  // resident blocks per CU of each (window variant, staging) kernel, 0 =
  // not yet known (matrix-core forms: [variant][0] plain, [variant][1] gate/up
  // pairs); a benign cache: every thread that fills it writes the same value
  mutable std::atomic<int> occupancy[5][3];   // by window variant and kernel (0 plain, 1 gate/up, 2 4-wave)
};

namespace {

// Enqueue fn with its by-value arguments and return the launch's own status
// (a stale error left by the caller's earlier HIP work is neither reported
// as the library's nor cleared).
template <class... A>
int enqueue(const void* fn, dim3 grid, dim3 block, size_t lds, void* stream, A... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(fn, grid, block, argv, lds, static_cast<hipStream_t>(stream)) == hipSuccess
             ? QGEMV_OK
             : QGEMV_E_HIP;
}

// Per-device facts, fetched once per device at the first launch on it:
// the compute-unit count, and every kernel's dynamic-LDS limit raised.
struct DeviceInfo {
  std::once_flag once;
  int cus = 0;
  int status = QGEMV_E_HIP;
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];

qg::StackKernels stack_kernels(int var) {
  switch (var) {
    case 0: return qg::stack_kernels_m1();
    case 1: return qg::stack_kernels_m2();
    case 2: return qg::stack_kernels_m4();
    case 3: return qg::stack_kernels_m8();
    default: return qg::stack_kernels_m16();
  }
}

void init_device(DeviceInfo* info) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return;
  for (int bi = 0; bi < 6; ++bi)
    for (int gi = 0; gi < 3; ++gi) {
      const qg::Entry& e = qg::entry(bi, gi);
      for (int v = 0; v < 5; ++v) {
        for (qg::KernelFn fn : {e.fast[v][0], e.fast[v][1], e.generic[v]})
          if (fn && hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                        hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(qg::kMaxDynamicLds)) != hipSuccess)
            return;
        const qg::WideEntry& we = qg::wide_entry(bi, gi);
        for (qg::KernelFn fn : {e.mfma[v], e.mfma_gateup[v], we.k[v], we.gateup[v], e.mfma_dyn[v], we.dyn[v],
                                v < 3 ? e.mfma_indexed[v] : nullptr, v < 3 ? e.mfma_gateup_indexed[v] : nullptr,
                                v < 3 ? we.indexed[v] : nullptr, v < 3 ? we.gateup_indexed[v] : nullptr})
          if (fn && hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(qg::kMaxMfmaLds)) != hipSuccess)
            return;
      }
    }
  for (int v = 0; v < 5; ++v) {
    const qg::StackKernels sk = stack_kernels(v);
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(sk.dot), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(qg::kMaxDynamicLds)) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(sk.mfma), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(qg::kMaxMfmaLds)) != hipSuccess)
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

// Both matrix-core forms share the load groups, K split, window passes and
// LDS plan; they differ only in how a round's products are formed.
bool matrix_cores(const qgemv_handle* h) {
  return h->arith == QGEMV_ARITH_MFMA || h->arith == QGEMV_ARITH_WIDE;
}

// The window variant of m rows: the narrowest that holds them, the widest
// (passes of 16 rows) beyond 16.
int window_variant(int m) {
  for (int i = 0; i < 5; ++i)
    if (m <= qg::kWindows[i]) return i;
  return 4;
}

// Dynamic LDS of one block: the staged window (activations and unit sums)
// plus, for the hand-off mode, one staging buffer per wave.
size_t lds_bytes(const qgemv_handle* h, int var, int stage) {
  const size_t mb = static_cast<size_t>(qg::kWindows[var]);
  const size_t k = static_cast<size_t>(h->d.k);
  if (!h->fast) return mb * (k / 32) * (64 + 4);
  const size_t eu = static_cast<size_t>(h->cpc < h->d.group ? h->cpc : h->d.group);
  size_t b = mb * (k * 2 + (k / eu) * 4);
  if (stage) b += static_cast<size_t>(qg::kWaves) * h->entry->fast_rows[var] * h->ppc * qg::kWave * 16;
  return b;
}

// The matrix-core kernels' LDS: the staged window (rows of k/32 units x 64
// bytes, a zero area of R * 256 bytes, unit sums; rows padded by 16 bytes),
// the routed list of an indexed call, and one load-group slot per wave (which
// also holds the wave's K-split partial sums at a tile's end).  Returns false
// when it exceeds one block's LDS.
bool mfma_plan(const qgemv_handle* h, int var, bool indexed, size_t* lds, int waves_override = 0) {
  const size_t mb = static_cast<size_t>(qg::kWindows[var]);
  const size_t units = static_cast<size_t>(h->d.k) / 32;
  const size_t waves = static_cast<size_t>(waves_override ? waves_override : h->entry->mfma_waves[var]);
  const size_t b = mb * (units * 64 + 16) + 256 * static_cast<size_t>(h->entry->mfma_group) + mb * (units + 4) * 4 +
                   (indexed ? qg::kMaxList * 4 : 0) + waves * h->entry->mfma_slot;
  if (b > qg::kMaxMfmaLds) return false;
  *lds = b;
  return true;
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

// The matrix-core form's K split as the kernels take it: its log2, the load
// groups of each part, and the rounded reciprocal of the 32-code units per
// row (the kernels split a staging index into row and unit with it).
void set_split(qg::Params& p, const qgemv_handle* h) {
  p.ksplit = h->ksplit;
  p.ks_shift = h->ksplit == 4 ? 2 : (h->ksplit == 2 ? 1 : 0);
  const int64_t units = h->d.k / 32;
  p.gpp = static_cast<int32_t>(units / (4 * static_cast<int64_t>(h->entry->mfma_group)) / h->ksplit);
  p.inv_units = 1.0f / static_cast<float>(units);
}

// up: the up matrix of a gate/up pair (matrix-core form), else nullptr.
int launch(const qgemv_handle* h, const uint16_t* x, int32_t m, float* y, int64_t ldy,
           const int32_t* idx, int32_t slots, int32_t epi, void* stream, size_t ybytes,
           const qgemv_handle* up = nullptr) {
  const DeviceInfo* dev = current_device();
  if (!dev) return QGEMV_E_HIP;
  const int indexed = idx != nullptr;
  int var = indexed ? window_variant(qg::kIndexedWindow) : window_variant(m);
  // hand-off staging for 3/5/6 bits when it fits; the direct mode gives the
  // same bits with more scattered loads
  int stage = (h->fast && h->ppc > 1) ? 1 : 0;
  if (stage && lds_bytes(h, var, 1) > qg::kMaxDynamicLds) stage = 0;
  const bool mfma = matrix_cores(h);
  const int own_var = var;   // the window's own variant, before any narrowing
  size_t lds = 0;
  if (mfma) {
    stage = 0;
    // A window too wide for one block's LDS runs as passes of a narrower
    // variant over the same tiles: each output of the matrix-core form
    // depends only on its own window row, so the bits are the same.
    while (!mfma_plan(h, var, indexed, &lds)) {
      if (var == 0) return QGEMV_E_WINDOW;
      --var;
    }
  } else {
    lds = lds_bytes(h, var, stage);
  }
  // Small matrices: a plain or strided call's 8- and 16-row windows of the
  // tile walk in blocks of 4 waves when blocks of 8 would cover at most half
  // the CUs, at the window's own variant when its 4-wave plan fits (a column's
  // arithmetic does not depend on its block: the same bits)
  static_assert(qg::kWindows[3] == 8 && qg::kWindows[4] == 16, "4-wave kernels for windows of 8 and 16 rows");
  bool four = false;
  if (mfma && !indexed && !up) {
    for (int v = own_var; v >= var && qg::kWindows[v] >= 8; --v) {
      const int64_t rows8 = static_cast<int64_t>(h->entry->mfma_waves[v] / h->ksplit) * 16;
      size_t l4 = 0;
      if (2 * ((h->d.n + rows8 - 1) / rows8) <= dev->cus && mfma_plan(h, v, false, &l4, 4)) {
        four = true;
        var = v;
        lds = l4;
        break;
      }
    }
  }
  if (lds > (mfma ? qg::kMaxMfmaLds : qg::kMaxDynamicLds)) return QGEMV_E_WINDOW;
  qg::KernelFn fn = h->fast ? h->entry->fast[var][stage] : h->entry->generic[var];
  int threads = qg::kThreads;
  int64_t tile_rows = 0;
  if (mfma) {
    // one wave per 16 output columns
    // gate/up pairs and indexed calls run kernels of their own, with the
    // pairing and the routing compiled in
    const bool wide = h->arith == QGEMV_ARITH_WIDE || (h->wide_windows && qg::kWindows[var] > 8 && !indexed);
    if (indexed) {
      if (var > 2) return QGEMV_E_WINDOW;   // routed windows have at most kIndexedWindow rows
      fn = wide ? (up ? h->wide->gateup_indexed[var] : h->wide->indexed[var])
                : (up ? h->entry->mfma_gateup_indexed[var] : h->entry->mfma_indexed[var]);
    } else {
      fn = wide ? (up ? h->wide->gateup[var] : (four ? h->wide->k4[var - 3] : h->wide->k[var]))
                : (up ? h->entry->mfma_gateup[var] : (four ? h->entry->mfma4[var - 3] : h->entry->mfma[var]));
    }
    const int nw = four ? 4 : h->entry->mfma_waves[var];
    threads = nw * qg::kWave;
    tile_rows = static_cast<int64_t>(nw / h->ksplit) * (up ? 8 : 16);
  } else {
    const int R = h->fast ? h->entry->fast_rows[var] : h->entry->generic_rows[var];
    const int slots_per_wave = qg::kWave / h->lpr;
    tile_rows = static_cast<int64_t>(qg::kWaves) * slots_per_wave * R;
  }
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
  p.vec_groups = h->vec_groups;
  set_split(p, h);
  p.gateup = up ? 1 : 0;
  p.w2 = up ? up->d.w : nullptr;
  p.scales2 = up ? up->d.scales : nullptr;
  p.biases2 = up ? up->d.biases : nullptr;
  p.y_bytes = static_cast<int64_t>(ybytes);
  p.nseg = 1;
  p.seg_row0[0] = 0;
  p.seg_delta[0] = 0;

  // A persistent grid: as many blocks as the CUs hold at once, each walking
  // its tiles with the staged window reused (grid size never changes bits:
  // a column's lanes and their arithmetic do not depend on its block).
  // (the matrix-core kernels always take staging 0: their slot 1 holds the
  // gate/up kernel's occupancy; indexed calls size their grid per expert)
  dim3 grid(1u, 1u);
  // A plain or strided call on a matrix of many 16-column units with no K
  // split: one block per CU, each CU's share of units handed out among its
  // waves (so that the CU's waves end together), when its kernel and LDS fit:
  // at the window's own variant (its block has fewer waves than the tile
  // walk's blocks together), else at the tile walk's narrower one (passes).
  // Its stages of one or two load groups need a row of whole stages, and its
  // loads of two groups' scales at once an 8- or 16-byte aligned scale array.
  const int64_t units16 = (h->d.n + 15) / 16;
  const uintptr_t sb_addr = reinterpret_cast<uintptr_t>(h->d.scales) | reinterpret_cast<uintptr_t>(h->d.biases);
  if (mfma && !indexed && !up && h->ksplit == 1 &&
      h->d.k % (128 * static_cast<int64_t>(h->entry->mfma_group) * h->entry->dyn_stage) == 0 &&
      sb_addr % static_cast<uintptr_t>(h->entry->dyn_salign) == 0) {
    for (int dv = own_var;; dv = var) {
      size_t dyn_lds = 0;
      const bool dyn_wide = h->arith == QGEMV_ARITH_WIDE || (h->wide_windows && qg::kWindows[dv] > 8);
      const int dyn_waves = qg::dyn_waves(h->d.bits, h->d.group, qg::kWindows[dv], dyn_wide);
      const qg::KernelFn dyn_fn = dyn_wide ? h->wide->dyn[dv] : h->entry->mfma_dyn[dv];
      if (dyn_fn && units16 >= 2LL * dyn_waves * dev->cus && mfma_plan(h, dv, false, &dyn_lds, dyn_waves)) {
        p.tiles = static_cast<int32_t>(units16);
        grid.x = static_cast<unsigned>(dev->cus);
        return enqueue(reinterpret_cast<const void*>(dyn_fn), grid, dim3(dyn_waves * qg::kWave), dyn_lds, stream,
                       p);
      }
      if (dv == var) break;
    }
  }
  if (!indexed) {
    const int oslot = mfma ? (up ? 1 : (four ? 2 : 0)) : stage;
    int occ = h->occupancy[var][oslot].load(std::memory_order_relaxed);
    if (occ == 0) {
      int nb = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(fn), threads,
                                                       lds) != hipSuccess || nb < 1)
        nb = 1;
      occ = nb;
      h->occupancy[var][oslot].store(occ, std::memory_order_relaxed);
    }
    int64_t blocks = tiles;
    const int64_t cap = static_cast<int64_t>(dev->cus) * occ;
    if (blocks > cap) blocks = cap;
    grid.x = static_cast<unsigned>(blocks);
  } else {
    // blocks per expert: enough that the experts a call routes to (not known
    // on the host) keep every CU's waves streaming, few enough that each
    // block's routing and window staging serve several tiles.  Measured on
    // MI355X (128 experts of 1024 x 2048, 16 rows x 8 slots): the matrix-core
    // form is fastest with 16 (4 tiles a block), the dot form with 32.  A
    // gate/up pair's tiles hold 8 output columns, twice as many tiles: 32
    // keeps 4 tiles a block.
    const int64_t most = mfma ? (up ? 32 : 16) : 32;
    const int64_t per = tiles < most ? tiles : most;
    grid.x = static_cast<unsigned>(per);
    grid.y = static_cast<unsigned>(h->d.n_experts);
  }
  return enqueue(reinterpret_cast<const void*>(fn), grid, dim3(threads), lds, stream, p);
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
    case QGEMV_E_INDEX: return "QGEMV_E_INDEX";
  }
  return "QGEMV_E_UNKNOWN";
}

int qgemv_create(const qgemv_desc* d, qgemv_t* out) { return qgemv_create_arith(d, QGEMV_ARITH_AUTO, out); }

int64_t qgemv_mfma_codes(int32_t bits, int32_t group) {
  const int bi = qg::bits_index(bits), gi = qg::group_index(group);
  if (bi < 0 || gi < 0) return 0;
  // one load group of 128-code rounds per step; with one round per group at
  // group 128 the scale loads take the aligned dword of two groups, so a row
  // holds an even number of groups
  const int64_t codes = 128 * static_cast<int64_t>(qg::entry(bi, gi).mfma_group);
  return (group == 128 && codes == 128) ? 256 : codes;
}

int qgemv_arith(qgemv_t h) { return h ? h->arith : QGEMV_E_ARG; }

int qgemv_create_arith(const qgemv_desc* d, int32_t arith, qgemv_t* out) {
  if (!d || !out) return QGEMV_E_ARG;
  if (arith != QGEMV_ARITH_AUTO && arith != QGEMV_ARITH_DOT && arith != QGEMV_ARITH_MFMA &&
      arith != QGEMV_ARITH_WIDE)
    return QGEMV_E_ARG;
  const int bi = qg::bits_index(d->bits);
  if (bi < 0) return QGEMV_E_BITS;
  const int gi = qg::group_index(d->group);
  if (gi < 0) return QGEMV_E_GROUP;
  if (d->n < 1 || d->k < 1 || d->k % d->group != 0 || (d->k * d->bits) % 32 != 0)
    return QGEMV_E_SHAPE;
  if (d->n_experts < 1) return QGEMV_E_SHAPE;
  // columns and tiles are int32 in the kernels, elements int64; one output
  // row must stay below 2 GiB
  if (d->n > (int64_t{1} << 28) || d->k > (int64_t{1} << 20) ||
      static_cast<double>(d->n) * d->k * d->n_experts > 1.0e12)
    return QGEMV_E_SHAPE;
  if (!d->w || !d->scales || !d->biases) return QGEMV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(d->w) & 15) || (reinterpret_cast<uintptr_t>(d->scales) & 1) ||
      (reinterpret_cast<uintptr_t>(d->biases) & 1))
    return QGEMV_E_ALIGN;

  std::unique_ptr<qgemv_handle> hp(new (std::nothrow) qgemv_handle());
  if (!hp) return QGEMV_E_ARG;
  qgemv_handle& h = *hp;
  for (auto& row : h.occupancy)
    for (auto& o : row) o.store(0);
  h.d = *d;
  h.wpr = d->k * d->bits / 32;
  h.gpr = d->k / d->group;
  h.entry = &qg::entry(bi, gi);
  h.wide = &qg::wide_entry(bi, gi);
  // Fast geometry when a row is a whole number of chunks and at least 16
  // lanes share a column; otherwise one 32-code unit per lane step.
  int ppc = 0, cpc = 0;
  qg::fast_geometry(d->bits, &ppc, &cpc);
  h.fast = 0;
  if (d->k % cpc == 0 && (d->k / cpc) % 16 == 0) {
    h.fast = 1;
    h.ppc = ppc;
    h.cpc = cpc;
  } else {
    h.ppc = 0;
    h.cpc = 32;
  }
  h.nchunks = static_cast<int>(d->k / h.cpc);
  int lpr = 1;
  while (lpr < 64 && h.nchunks % (lpr * 2) == 0) lpr *= 2;
  h.lpr = lpr;
  h.cpl = h.nchunks / lpr;
  // arithmetic: the matrix cores when asked for or when left to the library
  // and the shape allows them, else the dot form
  const uintptr_t sb = reinterpret_cast<uintptr_t>(d->scales) | reinterpret_cast<uintptr_t>(d->biases);
  const bool mfma_ok = d->k % qgemv_mfma_codes(d->bits, d->group) == 0 &&
                       sb % static_cast<uintptr_t>(h.entry->mfma_salign) == 0;
  if ((arith == QGEMV_ARITH_MFMA || arith == QGEMV_ARITH_WIDE) && !mfma_ok) return QGEMV_E_NOKERNEL;
  h.arith = arith == QGEMV_ARITH_WIDE ? QGEMV_ARITH_WIDE
            : (arith == QGEMV_ARITH_MFMA || (arith == QGEMV_ARITH_AUTO && mfma_ok)) ? QGEMV_ARITH_MFMA
                                                                                  : QGEMV_ARITH_DOT;
  // The two matrix-core forms give the same bits (the matrix cores sum a
  // 16x16x32 product's K as four 8-wide steps in order, so one product over
  // a unit equals the block-diagonal form's four chained products), so the
  // library's choice takes each window's faster kernels: block-diagonal up
  // to 8 rows, wide above.
  h.wide_windows = arith == QGEMV_ARITH_AUTO && h.arith == QGEMV_ARITH_MFMA;
  // matrix-core K split, from one expert's shape only (an indexed call must
  // give each expert the bits of that expert's own single-expert handle):
  // small matrices split K in 2 or 4 parts so that enough waves stream at
  // once (about 2048, two per SIMD), when the row's load groups divide evenly
  h.ksplit = 1;
  if (matrix_cores(&h)) {
    const int64_t groups = d->k / (128 * static_cast<int64_t>(h.entry->mfma_group));
    const int64_t col_tiles = (d->n + 15) / 16;
    while (h.ksplit < 4 && col_tiles * h.ksplit < 2048 && groups % (2 * h.ksplit) == 0) h.ksplit *= 2;
  }
  {
    // groups one packed scale load spans: a lane chunk's, or a 128-code
    // macro step's for the matrix-core form
    const int span_codes = matrix_cores(&h) ? 128 : h.cpc;
    const int gspan = span_codes >= d->group ? span_codes / d->group : 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(d->scales) | reinterpret_cast<uintptr_t>(d->biases);
    h.vec_groups = (a % (2 * gspan) == 0) && (h.gpr % gspan == 0);
  }
  // The one-row window must fit in LDS; wider windows are refused at run
  // time when theirs does not (QGEMV_E_WINDOW), or, in the matrix-core
  // form, run as passes of fewer rows.
  if (matrix_cores(&h)) {
    size_t lds = 0;
    if (!mfma_plan(&h, 0, false, &lds)) {
      if (arith == QGEMV_ARITH_MFMA || arith == QGEMV_ARITH_WIDE) return QGEMV_E_NOKERNEL;
      h.arith = QGEMV_ARITH_DOT;
      h.ksplit = 1;
      h.wide_windows = 0;
    }
  }
  if (h.arith == QGEMV_ARITH_DOT && lds_bytes(&h, 0, 0) > qg::kMaxDynamicLds) return QGEMV_E_SHAPE;
  *out = hp.release();
  return QGEMV_OK;
}

void qgemv_destroy(qgemv_t h) { delete h; }

// max_m: QGEMV_MAX_WINDOW, or for plain and strided calls on a matrix-core
// handle QGEMV_MAX_PROMPT (windows above 16 rows run as passes of 16)
static int check_run_common(qgemv_t h, const uint16_t* x, int32_t m, const float* y, int32_t epi,
                            int32_t max_m) {
  if (!h) return QGEMV_E_ARG;
  if (m < 0 || m > max_m) return QGEMV_E_WINDOW;
  if (epi != QGEMV_EPI_NONE && epi != QGEMV_EPI_RELU2) return QGEMV_E_ARG;
  if (m == 0) return QGEMV_OK;
  if (!x || !y) return QGEMV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 3)) return QGEMV_E_ALIGN;
  return QGEMV_OK;
}

int qgemv_run_strided(qgemv_t h, const uint16_t* x, int32_t m, float* y, int64_t ldy, int32_t epi,
                      void* stream) {
  int rc = check_run_common(h, x, m, y, epi,
                            h && matrix_cores(h) ? QGEMV_MAX_PROMPT : QGEMV_MAX_WINDOW);
  if (rc != QGEMV_OK) return rc;
  if (h->d.n_experts != 1) return QGEMV_E_ARG;
  if (ldy < h->d.n) return QGEMV_E_STRIDE;
  if (m == 0) return QGEMV_OK;
  const size_t xbytes = static_cast<size_t>(m) * h->d.k * 2;
  const size_t ybytes = (static_cast<size_t>(m - 1) * ldy + h->d.n) * 4;
  if (ybytes > static_cast<size_t>(qg::kNoOffset)) return QGEMV_E_STRIDE;
  rc = check_y_alias(h, y, ybytes, x, xbytes, nullptr, 0);
  if (rc != QGEMV_OK) return rc;
  return launch(h, x, m, y, ldy, nullptr, 0, epi, stream, ybytes);
}

int qgemv_run(qgemv_t h, const uint16_t* x, int32_t m, float* y, int32_t epi, void* stream) {
  if (!h) return QGEMV_E_ARG;
  return qgemv_run_strided(h, x, m, y, h->d.n, epi, stream);
}

int qgemv_run_indexed(qgemv_t h, const uint16_t* x, int32_t m, const int32_t* idx, int32_t slots,
                      float* y, int32_t epi, void* stream) {
  int rc = check_run_common(h, x, m, y, epi, QGEMV_MAX_WINDOW);
  if (rc != QGEMV_OK) return rc;
  if (slots < 0 || slots > qg::kMaxSlots) return QGEMV_E_ARG;
  if (m == 0 || slots == 0) return QGEMV_OK;
  if (!idx) return QGEMV_E_ARG;
  if (reinterpret_cast<uintptr_t>(idx) & 3) return QGEMV_E_ALIGN;
  const size_t xbytes = static_cast<size_t>(m) * h->d.k * 2;
  const size_t ybytes = static_cast<size_t>(m) * slots * h->d.n * 4;
  if (ybytes > static_cast<size_t>(qg::kNoOffset)) return QGEMV_E_SHAPE;
  rc = check_y_alias(h, y, ybytes, x, xbytes, idx, static_cast<size_t>(m) * slots * 4);
  if (rc != QGEMV_OK) return rc;
  return launch(h, x, m, y, h->d.n, idx, slots, epi, stream, ybytes);
}

int qgemv_check_indices(qgemv_t h, const int32_t* idx, int32_t m, int32_t slots, void* stream) {
  if (!h) return QGEMV_E_ARG;
  if (m < 0 || m > QGEMV_MAX_WINDOW) return QGEMV_E_WINDOW;
  if (slots < 0 || slots > qg::kMaxSlots) return QGEMV_E_ARG;
  if (m == 0 || slots == 0) return QGEMV_OK;
  if (!idx) return QGEMV_E_ARG;
  if (reinterpret_cast<uintptr_t>(idx) & 3) return QGEMV_E_ALIGN;
  int32_t host[QGEMV_MAX_WINDOW * qg::kMaxSlots];
  const size_t count = static_cast<size_t>(m) * slots;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host, idx, count * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return QGEMV_E_HIP;
  for (size_t i = 0; i < count; ++i)
    if (host[i] < 0 || host[i] >= h->d.n_experts) return QGEMV_E_INDEX;
  return QGEMV_OK;
}

static int check_gateup_pair(qgemv_t gate, qgemv_t up) {
  if (!gate || !up) return QGEMV_E_ARG;
  if (!matrix_cores(gate) || up->arith != gate->arith) return QGEMV_E_NOKERNEL;
  if (gate->d.bits != up->d.bits || gate->d.group != up->d.group || gate->d.n != up->d.n ||
      gate->d.k != up->d.k || gate->d.n_experts != up->d.n_experts || gate->ksplit != up->ksplit)
    return QGEMV_E_SHAPE;
  return QGEMV_OK;
}

int qgemv_run_gateup(qgemv_t gate, qgemv_t up, const uint16_t* x, int32_t m, float* y, int64_t ldy,
                     void* stream) {
  int rc = check_gateup_pair(gate, up);
  if (rc != QGEMV_OK) return rc;
  rc = check_run_common(gate, x, m, y, QGEMV_EPI_NONE, QGEMV_MAX_PROMPT);
  if (rc != QGEMV_OK) return rc;
  if (gate->d.n_experts != 1) return QGEMV_E_ARG;
  if (ldy < gate->d.n) return QGEMV_E_STRIDE;
  if (m == 0) return QGEMV_OK;
  const size_t xbytes = static_cast<size_t>(m) * gate->d.k * 2;
  const size_t ybytes = (static_cast<size_t>(m - 1) * ldy + gate->d.n) * 4;
  if (ybytes > static_cast<size_t>(qg::kNoOffset)) return QGEMV_E_STRIDE;
  rc = check_y_alias(gate, y, ybytes, x, xbytes, nullptr, 0);
  if (rc == QGEMV_OK) rc = check_y_alias(up, y, ybytes, x, xbytes, nullptr, 0);
  if (rc != QGEMV_OK) return rc;
  return launch(gate, x, m, y, ldy, nullptr, 0, QGEMV_EPI_NONE, stream, ybytes, up);
}

int qgemv_run_gateup_indexed(qgemv_t gate, qgemv_t up, const uint16_t* x, int32_t m, const int32_t* idx,
                             int32_t slots, float* y, void* stream) {
  int rc = check_gateup_pair(gate, up);
  if (rc != QGEMV_OK) return rc;
  rc = check_run_common(gate, x, m, y, QGEMV_EPI_NONE, QGEMV_MAX_WINDOW);
  if (rc != QGEMV_OK) return rc;
  if (slots < 0 || slots > qg::kMaxSlots) return QGEMV_E_ARG;
  if (m == 0 || slots == 0) return QGEMV_OK;
  if (!idx) return QGEMV_E_ARG;
  if (reinterpret_cast<uintptr_t>(idx) & 3) return QGEMV_E_ALIGN;
  const size_t xbytes = static_cast<size_t>(m) * gate->d.k * 2;
  const size_t ybytes = static_cast<size_t>(m) * slots * gate->d.n * 4;
  if (ybytes > static_cast<size_t>(qg::kNoOffset)) return QGEMV_E_SHAPE;
  const size_t ib = static_cast<size_t>(m) * slots * 4;
  rc = check_y_alias(gate, y, ybytes, x, xbytes, idx, ib);
  if (rc == QGEMV_OK) rc = check_y_alias(up, y, ybytes, x, xbytes, idx, ib);
  if (rc != QGEMV_OK) return rc;
  return launch(gate, x, m, y, gate->d.n, idx, slots, QGEMV_EPI_NONE, stream, ybytes, up);
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
  return enqueue(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(blocks)), dim3(qg::kThreads), 0,
                 stream, w, n, k, codes);
}


int qgemv_common_width(const int32_t* bits, const int32_t* groups, int32_t count, int32_t* bits_out,
                       int32_t* group_out) {
  if (!bits || !groups || !bits_out || !group_out || count < 1) return QGEMV_E_ARG;
  int32_t b = 0, g = 1 << 30;
  for (int32_t i = 0; i < count; ++i) {
    if (qg::bits_index(bits[i]) < 0) return QGEMV_E_BITS;
    if (qg::group_index(groups[i]) < 0) return QGEMV_E_GROUP;
    if (bits[i] > b) b = bits[i];
    if (groups[i] < g) g = groups[i];
  }
  *bits_out = b;
  *group_out = g;
  return QGEMV_OK;
}

int qgemv_widen(const qgemv_desc* src, int32_t bits_out, int32_t group_out, uint32_t* w_out, uint16_t* scales_out,
                uint16_t* biases_out, void* stream) {
  if (!src || !w_out || !scales_out || !biases_out) return QGEMV_E_ARG;
  // the source is admitted exactly as qgemv_create admits it
  qgemv_t probe = nullptr;
  const int rc = qgemv_create(src, &probe);
  if (rc != QGEMV_OK) return rc;
  qgemv_destroy(probe);
  if (qg::bits_index(bits_out) < 0 || bits_out < src->bits) return QGEMV_E_BITS;
  if (qg::group_index(group_out) < 0 || src->group % group_out != 0) return QGEMV_E_GROUP;
  if (reinterpret_cast<uintptr_t>(w_out) & 15 || reinterpret_cast<uintptr_t>(scales_out) & 1 ||
      reinterpret_cast<uintptr_t>(biases_out) & 1)
    return QGEMV_E_ALIGN;
  const int64_t rows = src->n * src->n_experts;
  const int64_t units = rows * (src->k / 32);
  const int64_t groups_out = rows * (src->k / group_out);
  const size_t in_w = static_cast<size_t>(units) * src->bits * 4, out_w = static_cast<size_t>(units) * bits_out * 4;
  const size_t in_s = static_cast<size_t>(rows) * (src->k / src->group) * 2, out_s = static_cast<size_t>(groups_out) * 2;
  for (const void* o : {static_cast<const void*>(w_out), static_cast<const void*>(scales_out),
                        static_cast<const void*>(biases_out)}) {
    const size_t ob = o == w_out ? out_w : out_s;
    if (overlaps(o, ob, src->w, in_w) || overlaps(o, ob, src->scales, in_s) || overlaps(o, ob, src->biases, in_s))
      return QGEMV_E_ALIAS;
  }
  if (overlaps(w_out, out_w, scales_out, out_s) || overlaps(w_out, out_w, biases_out, out_s) ||
      overlaps(scales_out, out_s, biases_out, out_s))
    return QGEMV_E_ALIAS;
  if (!current_device()) return QGEMV_E_HIP;
  const int ratio = src->group / group_out;
  int rc2 = enqueue(reinterpret_cast<const void*>(qg::widen_kernel),
                    dim3(static_cast<unsigned>((units + qg::kThreads - 1) / qg::kThreads)), dim3(qg::kThreads), 0,
                    stream, src->w, static_cast<int>(src->bits), w_out, static_cast<int>(bits_out), units);
  const unsigned gb = static_cast<unsigned>((groups_out + qg::kThreads - 1) / qg::kThreads);
  if (rc2 == QGEMV_OK)
    rc2 = enqueue(reinterpret_cast<const void*>(qg::regroup_kernel), dim3(gb), dim3(qg::kThreads), 0, stream,
                  src->scales, static_cast<uint16_t*>(scales_out), ratio, groups_out);
  if (rc2 == QGEMV_OK)
    rc2 = enqueue(reinterpret_cast<const void*>(qg::regroup_kernel), dim3(gb), dim3(qg::kThreads), 0, stream,
                  src->biases, static_cast<uint16_t*>(biases_out), ratio, groups_out);
  return rc2;
}

struct qgemv_stack {
  int n_runs;
  int64_t ldy;
  int64_t col_end;                       // one past the last member column
  qgemv_handle* run[qg::kMaxRuns];
  int n_members[qg::kMaxRuns];
  int64_t member_rows[qg::kMaxRuns][qg::kMaxSeg];
  int64_t member_cols[qg::kMaxRuns][qg::kMaxSeg];
  mutable std::atomic<int> occupancy[5][2];   // by window variant and form (0 dot, 1 matrix-core)
  ~qgemv_stack() {
    for (int r = 0; r < n_runs; ++r) delete run[r];
  }
};

int qgemv_stack_create(const qgemv_run_spec* runs, int32_t n_runs, int64_t ldy, qgemv_stack_t* out) {
  if (!runs || !out) return QGEMV_E_ARG;
  if (n_runs < 1 || n_runs > qg::kMaxRuns) return QGEMV_E_ARG;
  if (ldy < 1) return QGEMV_E_STRIDE;
  std::unique_ptr<qgemv_stack> st(new (std::nothrow) qgemv_stack());
  if (!st) return QGEMV_E_ARG;
  for (auto& row : st->occupancy)
    for (auto& o : row) o.store(0);
  st->ldy = ldy;
  st->n_runs = 0;
  int64_t ranges[qg::kMaxRuns * qg::kMaxSeg][2];
  int nranges = 0;
  for (int r = 0; r < n_runs; ++r) {
    const qgemv_run_spec& rr = runs[r];
    qgemv_t h = nullptr;
    const int rc = qgemv_create(&rr.w, &h);
    if (rc != QGEMV_OK) return rc;
    st->run[st->n_runs++] = h;
    if (rr.w.n_experts != 1) return QGEMV_E_ARG;
    if (rr.w.k != runs[0].w.k) return QGEMV_E_SHAPE;
    if (h->arith == QGEMV_ARITH_DOT && !h->fast) return QGEMV_E_NOKERNEL;
    if (rr.n_members < 1 || rr.n_members > qg::kMaxSeg) return QGEMV_E_ARG;
    int64_t rows = 0;
    for (int mbr = 0; mbr < rr.n_members; ++mbr) {
      const int64_t nr = rr.member_rows[mbr], c = rr.member_cols[mbr];
      if (nr < 1) return QGEMV_E_SHAPE;
      if (c < 0 || c + nr > ldy) return QGEMV_E_STRIDE;
      for (int q = 0; q < nranges; ++q)
        if (c < ranges[q][1] && ranges[q][0] < c + nr) return QGEMV_E_ALIAS;
      ranges[nranges][0] = c;
      ranges[nranges][1] = c + nr;
      ++nranges;
      st->member_rows[r][mbr] = nr;
      st->member_cols[r][mbr] = c;
      if (c + nr > st->col_end) st->col_end = c + nr;
      rows += nr;
    }
    if (rows != rr.w.n) return QGEMV_E_SHAPE;
    st->n_members[r] = rr.n_members;
  }
  *out = st.release();
  return QGEMV_OK;
}

void qgemv_stack_destroy(qgemv_stack_t s) { delete s; }

}  // extern "C"

namespace {

// One dispatch over the runs of a stack that share an arithmetic form.
int launch_stack(const qgemv_stack* s, bool mfma, const uint16_t* x, int32_t m, float* y, int32_t epi,
                 void* stream, size_t ybytes, const DeviceInfo* dev) {
  int idx[qg::kMaxRuns];
  int nr = 0;
  for (int r = 0; r < s->n_runs; ++r)
    if ((s->run[r]->arith == QGEMV_ARITH_MFMA) == mfma) idx[nr++] = r;
  if (nr == 0) return QGEMV_OK;
  // grid rows in order of a block's serial work (its wave's codes times
  // their width), longest first: the hardware places blocks in launch order,
  // so the blocks that bound the dispatch get CUs of their own when the
  // runs together have more blocks than there are CUs
  auto work = [&](int r) {
    const qgemv_handle* h = s->run[r];
    return (h->d.k / (h->arith == QGEMV_ARITH_DOT ? 1 : h->ksplit)) * h->d.bits;
  };
  for (int a = 1; a < nr; ++a)
    for (int b = a; b > 0 && work(idx[b]) > work(idx[b - 1]); --b) std::swap(idx[b], idx[b - 1]);
  int var = window_variant(m);
  size_t lds = 0;
  if (mfma) {
    // the widest variant whose LDS every run fits (narrower ones run the
    // window as passes, same bits)
    for (;; --var) {
      lds = 0;
      bool fits = true;
      for (int q = 0; q < nr && fits; ++q) {
        size_t l = 0;
        fits = mfma_plan(s->run[idx[q]], var, false, &l);
        if (l > lds) lds = l;
      }
      if (fits) break;
      if (var == 0) return QGEMV_E_WINDOW;
    }
  }
  qg::StackParams sp{};
  sp.nruns = nr;
  int64_t tiles[qg::kMaxRuns];
  int64_t total_tiles = 0;
  int threads = qg::kThreads;
  for (int q = 0; q < nr; ++q) {
    const int r = idx[q];
    const qgemv_handle* h = s->run[r];
    const int bi = qg::bits_index(h->d.bits), gi = qg::group_index(h->d.group);
    int64_t tile_rows = 0;
    if (mfma) {
      threads = h->entry->mfma_waves[var] * qg::kWave;
      tile_rows = static_cast<int64_t>(h->entry->mfma_waves[var] / h->ksplit) * 16;
      sp.sel[q].kind = bi * 3 + gi;
    } else {
      int stage = h->ppc > 1 ? 1 : 0;
      if (stage && lds_bytes(h, var, 1) > qg::kMaxDynamicLds) stage = 0;
      const size_t l = lds_bytes(h, var, stage);
      if (l > qg::kMaxDynamicLds) return QGEMV_E_WINDOW;
      if (l > lds) lds = l;
      const int R = h->entry->fast_rows[var];
      tile_rows = static_cast<int64_t>(qg::kWaves) * (qg::kWave / h->lpr) * R;
      sp.sel[q].kind = (bi * 3 + gi) * 2 + stage;
    }
    tiles[q] = (h->d.n + tile_rows - 1) / tile_rows;
    total_tiles += tiles[q];
    qg::Params& p = sp.run[q];
    p.w = h->d.w;
    p.scales = h->d.scales;
    p.biases = h->d.biases;
    p.x = x;
    p.y = y;
    p.idx = nullptr;
    p.n = h->d.n;
    p.k = h->d.k;
    p.wpr = h->wpr;
    p.gpr = h->gpr;
    p.ldy = s->ldy;
    p.m = m;
    p.slots = 0;
    p.n_experts = 1;
    p.epi = epi;
    p.lpr = h->lpr;
    p.cpl = h->cpl;
    p.nchunks = h->nchunks;
    p.tiles = static_cast<int32_t>(tiles[q]);
    p.indexed = 0;
    p.vec_groups = h->vec_groups;
    set_split(p, h);
    p.y_bytes = static_cast<int64_t>(ybytes);
    p.nseg = s->n_members[r];
    int64_t row0 = 0;
    for (int mbr = 0; mbr < s->n_members[r]; ++mbr) {
      p.seg_row0[mbr] = static_cast<int32_t>(row0);
      p.seg_delta[mbr] = s->member_cols[r][mbr] - row0;
      row0 += s->member_rows[r][mbr];
    }
  }
  const qg::StackKernels sk = stack_kernels(var);
  const qg::StackFn fn = mfma ? sk.mfma : sk.dot;
  int occ = s->occupancy[var][mfma].load(std::memory_order_relaxed);
  if (occ == 0) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(fn), threads, lds) !=
            hipSuccess || nb < 1)
      nb = 1;
    occ = nb;
    s->occupancy[var][mfma].store(occ, std::memory_order_relaxed);
  }
  // blocks per run: every tile its own block when the CUs hold them all,
  // else a share of the resident blocks in proportion to the run's tiles.
  // Grid row q holds run q's blocks; a row's blocks past its run's count
  // leave at once.
  const int64_t cap = static_cast<int64_t>(dev->cus) * occ;
  int64_t widest = 1;
  for (int q = 0; q < nr; ++q) {
    int64_t nb = tiles[q];
    if (total_tiles > cap) {
      nb = cap * tiles[q] / total_tiles;
      if (nb < 1) nb = 1;
      if (nb > tiles[q]) nb = tiles[q];
    }
    sp.sel[q].nblocks = static_cast<int32_t>(nb);
    if (nb > widest) widest = nb;
  }
  return enqueue(reinterpret_cast<const void*>(fn), dim3(static_cast<unsigned>(widest), static_cast<unsigned>(nr)),
                 dim3(threads), lds, stream, sp);
}

}  // namespace

extern "C" {

int qgemv_stack_run(qgemv_stack_t s, const uint16_t* x, int32_t m, float* y, int32_t epi, void* stream) {
  if (!s) return QGEMV_E_ARG;
  if (m < 0 || m > QGEMV_MAX_WINDOW) return QGEMV_E_WINDOW;
  if (epi != QGEMV_EPI_NONE && epi != QGEMV_EPI_RELU2) return QGEMV_E_ARG;
  if (m == 0) return QGEMV_OK;
  if (!x || !y) return QGEMV_E_ARG;
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 3)) return QGEMV_E_ALIGN;
  const int64_t k = s->run[0]->d.k;
  const size_t xbytes = static_cast<size_t>(m) * k * 2;
  const size_t ybytes = (static_cast<size_t>(m - 1) * s->ldy + s->col_end) * 4;
  if (ybytes > static_cast<size_t>(qg::kNoOffset)) return QGEMV_E_STRIDE;
  for (int r = 0; r < s->n_runs; ++r) {
    const int rc = check_y_alias(s->run[r], y, ybytes, x, xbytes, nullptr, 0);
    if (rc != QGEMV_OK) return rc;
  }
  const DeviceInfo* dev = current_device();
  if (!dev) return QGEMV_E_HIP;
  // one dispatch per arithmetic form present (one, unless some run's shape
  // rules out the matrix cores)
  int rc = launch_stack(s, true, x, m, y, epi, stream, ybytes, dev);
  if (rc != QGEMV_OK) return rc;
  return launch_stack(s, false, x, m, y, epi, stream, ybytes, dev);
}

int qgemv_query(qgemv_t h, int64_t out[6]) {
  if (!h || !out) return QGEMV_E_ARG;
  if (matrix_cores(h)) {
    // four lanes per column (one 32-code unit each), 16 columns per wave
    out[0] = 4;
    out[1] = 16;
    out[2] = 32;
    out[3] = h->entry->mfma_waves[0] * qg::kWave;
    out[4] = static_cast<int64_t>(h->entry->mfma_waves[0] / h->ksplit) * 16;
  } else {
    const int R = h->fast ? h->entry->fast_rows[0] : h->entry->generic_rows[0];
    out[0] = h->lpr;
    out[1] = (qg::kWave / h->lpr) * R;
    out[2] = h->cpc;
    out[3] = qg::kThreads;
    out[4] = static_cast<int64_t>(qg::kWaves) * (qg::kWave / h->lpr) * R;
  }
  const DeviceInfo* dev = current_device();
  out[5] = dev ? dev->cus : 0;
  return QGEMV_OK;
}

}  // extern "C"
