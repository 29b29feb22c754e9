// commit.hip -- the commit step after verify on gfx950: each batch row's state after its last consumed
// token is gathered from the per-position verify-state buffer into the row's cache slot, for every
// stateful tensor stacked across layers, and the row's sequence length advances by accept_len
// (AReno pull request "feat(engine): MTP training loss and speculative decoding for bailing_v3", section
// "What does this PR do?": the Phase-2 paragraph and the per-step table's commit row).
//
// The work is a pure HBM stream (every byte read once, written once), so the kernel is laid out for
// bandwidth: 128-thread workgroups copy 4 KiB tiles with 128-bit loads, a thread's two loads issued
// before its stores.  Rows of at least one tile get tiles that never cross a row (the tile's source and
// destination addresses are workgroup-uniform scalars); smaller rows are packed several to a tile, each
// lane finding its row by division.  One launch covers every tensor.  Loads go through the caches (a
// verify buffer the forward has just written may still sit in the 256 MB Infinity Cache), stores are
// nontemporal (the cache rows are not read again before the next step).  Measured on the hybrid-model
// stand-in (0.8 GB each way), this shape beat 256- and 512-thread groups, 8/16/32 KiB tiles, persistent
// grids and nontemporal loads, and a plain device copy of the same bytes.
#include "specverify.h"
#include "sv_common.h"

#include <cstring>

namespace sv {
namespace commit {

constexpr int CT = 128;   // threads per workgroup
constexpr int UNR = 2;    // units per thread per tile
constexpr int TU = CT * UNR;
constexpr uint32_t MAXGRID = 1u << 20;

struct TensorArg {
  const uint8_t* src;   // [L, B, k+1, row_bytes]
  uint8_t* dst;         // [L, num_slots, row_bytes]
  uint64_t row_bytes;
  uint64_t tile0;       // first tile of this tensor in the launch
  uint64_t nunits;      // L * B * nu (packed mode)
  uint32_t L;
  uint32_t nu;          // units of `unit` bytes per row
  uint32_t unit;        // 16, 4 or 1
  uint32_t tpr;         // tiles per row in row mode; 0 = packed mode
};

struct CommitParams {
  TensorArg t[SPEC_COMMIT_MAX_TENSORS];
  const int32_t* slot;
  const int32_t* acc;
  int32_t* seq_len;
  int32_t* status;
  uint64_t ntiles;      // tiles over all tensors
  int32_t n;
  int32_t B;
  int32_t k;
  int32_t num_slots;
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class U> struct Unit;
template <> struct Unit<u32x4> { static constexpr uint32_t BYTES = 16; };
template <> struct Unit<uint32_t> { static constexpr uint32_t BYTES = 4; };
template <> struct Unit<uint8_t> { static constexpr uint32_t BYTES = 1; };

// Byte offsets of row b's committed source state and its slot, or false if the row is not committed.
__device__ __forceinline__ bool row_ends(const CommitParams& p, uint32_t l, uint32_t b, uint64_t rb,
                                         uint64_t& from, uint64_t& to) {
  const int32_t a = p.acc[b];
  const int32_t s = p.slot[b];
  if (a < 1 || a > p.k + 1 || s < 0 || s >= p.num_slots) return false;
  from = (((uint64_t)l * (uint32_t)p.B + b) * (uint64_t)(p.k + 1) + (uint64_t)(a - 1)) * rb;
  to = ((uint64_t)l * (uint32_t)p.num_slots + (uint32_t)s) * rb;
  return true;
}

// A tile inside one row: units [chunk * TU, min(nu, (chunk + 1) * TU)) of row segment `seg` = l * B + b.
template <class U>
__device__ __forceinline__ void row_tile(const CommitParams& p, const TensorArg& t, uint64_t rel) {
  const uint32_t seg = (uint32_t)(rel / t.tpr);
  const uint32_t chunk = (uint32_t)(rel - (uint64_t)seg * t.tpr);
  const uint32_t l = seg / (uint32_t)p.B;
  const uint32_t b = seg - l * (uint32_t)p.B;
  uint64_t from, to;
  if (!row_ends(p, l, b, t.row_bytes, from, to)) return;
  const U* src = (const U*)(t.src + from);
  U* dst = (U*)(t.dst + to);
  const uint32_t u0 = chunk * (uint32_t)TU + threadIdx.x;
  U v[UNR];
#pragma unroll
  for (int j = 0; j < UNR; ++j) {
    const uint32_t u = u0 + j * CT;
    if (u < t.nu) v[j] = src[u];
  }
#pragma unroll
  for (int j = 0; j < UNR; ++j) {
    const uint32_t u = u0 + j * CT;
    if (u < t.nu) __builtin_nontemporal_store(v[j], dst + u);
  }
}

// A tile of TU consecutive units of the tensor's rows laid end to end (rows shorter than a tile).
template <class U>
__device__ __forceinline__ void packed_tile(const CommitParams& p, const TensorArg& t, uint64_t rel) {
  const uint64_t g0 = rel * (uint64_t)TU;
  const uint64_t s0 = g0 / t.nu;                      // first row segment of the tile
  const uint32_t o0 = (uint32_t)(g0 - s0 * t.nu);
  U v[UNR];
  uint64_t dsto[UNR];
#pragma unroll
  for (int j = 0; j < UNR; ++j) {
    dsto[j] = ~0ull;
    if (g0 + j * CT + threadIdx.x >= t.nunits) continue;
    const uint32_t r = o0 + j * CT + threadIdx.x;     // < nu + TU
    const uint32_t ds = r / t.nu;
    const uint32_t off = r - ds * t.nu;
    const uint32_t seg = (uint32_t)s0 + ds;
    const uint32_t l = seg / (uint32_t)p.B;
    const uint32_t b = seg - l * (uint32_t)p.B;
    uint64_t from, to;
    if (!row_ends(p, l, b, t.row_bytes, from, to)) continue;
    v[j] = *(const U*)(t.src + from + (uint64_t)off * Unit<U>::BYTES);
    dsto[j] = to + (uint64_t)off * Unit<U>::BYTES;
  }
#pragma unroll
  for (int j = 0; j < UNR; ++j)
    if (dsto[j] != ~0ull) *(U*)(t.dst + dsto[j]) = v[j];
}

template <class U>
__device__ __forceinline__ void do_tile(const CommitParams& p, const TensorArg& t, uint64_t rel) {
  if (t.tpr) row_tile<U>(p, t, rel);
  else packed_tile<U>(p, t, rel);
}

__global__ __launch_bounds__(CT) void k_commit(const CommitParams p) {
  // row bookkeeping: status and sequence length, one lane per row
  for (uint32_t b = blockIdx.x * CT + threadIdx.x; b < (uint32_t)p.B; b += gridDim.x * CT) {
    const int32_t a = p.acc[b];
    const int32_t s = p.slot[b];
    const int32_t st = (a < 1 || a > p.k + 1) ? 1 : (s < 0 || s >= p.num_slots) ? 2 : 0;
    if (p.status) p.status[b] = st;
    if (st == 0 && p.seq_len) p.seq_len[b] += a;
  }
  for (uint64_t tile = blockIdx.x; tile < p.ntiles; tile += gridDim.x) {
    int ti = 0;
    while (ti + 1 < p.n && tile >= p.t[ti + 1].tile0) ++ti;
    const TensorArg& t = p.t[ti];
    const uint64_t rel = tile - t.tile0;
    if (t.unit == 16) do_tile<u32x4>(p, t, rel);
    else if (t.unit == 4) do_tile<uint32_t>(p, t, rel);
    else do_tile<uint8_t>(p, t, rel);
  }
}

// Commit by slot numbers: one lane per row swaps the row's committed slot with the slot that holds the
// state after its accepted position.
__global__ __launch_bounds__(256) void k_commit_slots(int32_t* __restrict__ state_slot, int32_t* __restrict__ pos_slot,
                                                      const int32_t* __restrict__ acc, int32_t* __restrict__ seq_len,
                                                      int32_t* __restrict__ status, int32_t B, int32_t k,
                                                      int32_t num_slots) {
  const uint32_t b = blockIdx.x * 256u + threadIdx.x;
  if (b >= (uint32_t)B) return;
  const int32_t a = acc[b];
  int32_t st = 1;
  if (a >= 1 && a <= k + 1) {
    const size_t j = (size_t)b * (size_t)(k + 1) + (size_t)(a - 1);
    const int32_t cur = state_slot[b];
    const int32_t nxt = pos_slot[j];
    st = (cur < 0 || cur >= num_slots || nxt < 0 || nxt >= num_slots) ? 2 : 0;
    if (st == 0) {
      state_slot[b] = nxt;
      pos_slot[j] = cur;
      if (seq_len) seq_len[b] += a;
    }
  }
  if (status) status[b] = st;
}

static bool overlap(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb) { return a < b + nb && b < a + na; }

}  // namespace commit
}  // namespace sv

using namespace sv::commit;

extern "C" spec_status_t spec_commit(const spec_state_tensor_t* tensors, int32_t n_tensors, const int32_t* state_slot,
                                     const int32_t* accept_len, int32_t* seq_len, int32_t* status, int32_t B,
                                     int32_t k, int32_t num_slots, void* stream) {
  if (B < 1 || B > (1 << 20) || k < 0 || k > 255 || num_slots < 1) return SPEC_ERR_INVALID_ARGUMENT;
  if (n_tensors < 0 || n_tensors > SPEC_COMMIT_MAX_TENSORS || (n_tensors > 0 && !tensors))
    return SPEC_ERR_INVALID_ARGUMENT;
  if (!state_slot || !accept_len) return SPEC_ERR_INVALID_ARGUMENT;
  {  // the per-row outputs must not alias the per-row inputs
    const uint64_t rb = (uint64_t)B * 4;
    for (const int32_t* o : {(const int32_t*)seq_len, (const int32_t*)status})
      if (o && (overlap((uintptr_t)o, rb, (uintptr_t)state_slot, rb) ||
                overlap((uintptr_t)o, rb, (uintptr_t)accept_len, rb)))
        return SPEC_ERR_INVALID_ARGUMENT;
    if (seq_len && status && overlap((uintptr_t)seq_len, rb, (uintptr_t)status, rb)) return SPEC_ERR_INVALID_ARGUMENT;
  }
  CommitParams p;
  std::memset(&p, 0, sizeof(p));
  p.slot = state_slot;
  p.acc = accept_len;
  p.seq_len = seq_len;
  p.status = status;
  p.n = n_tensors;
  p.B = B;
  p.k = k;
  p.num_slots = num_slots;
  uint64_t tiles = 0;
  uintptr_t lo[2 * SPEC_COMMIT_MAX_TENSORS];
  uint64_t len[2 * SPEC_COMMIT_MAX_TENSORS];
  for (int i = 0; i < n_tensors; ++i) {
    const spec_state_tensor_t& d = tensors[i];
    if (!d.verify_state || !d.state_cache || d.row_bytes < 1 || d.layers < 1) return SPEC_ERR_INVALID_ARGUMENT;
    if ((int64_t)d.layers * B >= (1ll << 31)) return SPEC_ERR_INVALID_ARGUMENT;
    const uint64_t rb = (uint64_t)d.row_bytes;
    const uintptr_t s = (uintptr_t)d.verify_state, c = (uintptr_t)d.state_cache;
    uint32_t unit = 1;
    if (rb % 16 == 0 && s % 16 == 0 && c % 16 == 0) unit = 16;
    else if (rb % 4 == 0 && s % 4 == 0 && c % 4 == 0) unit = 4;
    if (rb / unit >= (1ull << 31) - TU) return SPEC_ERR_INVALID_ARGUMENT;
    // byte extents (overflow-checked): verify L*B*(k+1)*rb, cache L*num_slots*rb
    const uint64_t vrows = (uint64_t)d.layers * (uint64_t)B * (uint64_t)(k + 1);
    const uint64_t crows = (uint64_t)d.layers * (uint64_t)num_slots;
    if (rb > (~0ull >> 2) / vrows || rb > (~0ull >> 2) / crows) return SPEC_ERR_INVALID_ARGUMENT;
    lo[2 * i] = s;
    len[2 * i] = vrows * rb;
    lo[2 * i + 1] = c;
    len[2 * i + 1] = crows * rb;
    TensorArg& t = p.t[i];
    t.src = (const uint8_t*)d.verify_state;
    t.dst = (uint8_t*)d.state_cache;
    t.row_bytes = rb;
    t.L = (uint32_t)d.layers;
    t.unit = unit;
    t.nu = (uint32_t)(rb / unit);
    t.nunits = (uint64_t)d.layers * (uint64_t)B * t.nu;
    t.tile0 = tiles;
    if (t.nu >= (uint32_t)TU) {
      t.tpr = (t.nu + TU - 1) / TU;
      tiles += (uint64_t)d.layers * (uint64_t)B * t.tpr;
    } else {
      t.tpr = 0;
      tiles += (t.nunits + TU - 1) / TU;
    }
  }
  // no verify buffer may overlap a cache, and no two caches may overlap
  for (int i = 0; i < n_tensors; ++i)
    for (int j = 0; j < n_tensors; ++j) {
      if (overlap(lo[2 * i], len[2 * i], lo[2 * j + 1], len[2 * j + 1])) return SPEC_ERR_INVALID_ARGUMENT;
      if (i < j && overlap(lo[2 * i + 1], len[2 * i + 1], lo[2 * j + 1], len[2 * j + 1]))
        return SPEC_ERR_INVALID_ARGUMENT;
    }
  p.ntiles = tiles;
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || !sv::device_ok(dev, cus)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  const uint64_t status_wgs = ((uint64_t)B + CT - 1) / CT;
  uint64_t grid = tiles > status_wgs ? tiles : status_wgs;
  if (grid > MAXGRID) grid = MAXGRID;
  (void)hipGetLastError();  // an earlier runtime call's error would otherwise be taken for this launch's
  hipLaunchKernelGGL(k_commit, dim3((unsigned)grid), dim3(CT), 0, (hipStream_t)stream, p);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}

extern "C" spec_status_t spec_commit_slots(int32_t* state_slot, int32_t* pos_slot, const int32_t* accept_len,
                                           int32_t* seq_len, int32_t* status, int32_t B, int32_t k, int32_t num_slots,
                                           void* stream) {
  if (B < 1 || B > (1 << 20) || k < 0 || k > 255 || num_slots < 1) return SPEC_ERR_INVALID_ARGUMENT;
  if (!state_slot || !pos_slot || !accept_len) return SPEC_ERR_INVALID_ARGUMENT;
  // no two of the per-row arrays may overlap
  const uintptr_t p[5] = {(uintptr_t)state_slot, (uintptr_t)pos_slot, (uintptr_t)accept_len, (uintptr_t)seq_len,
                          (uintptr_t)status};
  const uint64_t n[5] = {(uint64_t)B * 4, (uint64_t)B * (uint64_t)(k + 1) * 4, (uint64_t)B * 4, (uint64_t)B * 4,
                         (uint64_t)B * 4};
  for (int i = 0; i < 5; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (p[i] && p[j] && overlap(p[i], n[i], p[j], n[j])) return SPEC_ERR_INVALID_ARGUMENT;
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || !sv::device_ok(dev, cus)) return SPEC_ERR_UNSUPPORTED_DEVICE;
  (void)hipGetLastError();  // an earlier runtime call's error would otherwise be taken for this launch's
  hipLaunchKernelGGL(k_commit_slots, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, (hipStream_t)stream, state_slot,
                     pos_slot, accept_len, seq_len, status, B, k, num_slots);
  if (hipGetLastError() != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}
