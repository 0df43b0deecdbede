// Hybrid-batch attention kernels for gfx950 (CDNA4): prefill tile, split-KV
// decode, last-arriver merge, and the fused launcher that picks each
// workgroup's role from the compute unit it landed on.
//
// Method (POD-Attention): prefill attention is compute-bound and decode
// attention bandwidth-bound (paper abstract; §1), so one launch should run
// both on every compute unit at once (§4).  A regular grid is launched and
// every workgroup is remapped to a virtual prefill or decode workgroup
// (§4.3); the choice is made after dispatch from what already runs on the
// workgroup's compute unit (§4.1 SM-aware CTA scheduling: by default a
// per-CU count of running prefill and decode workgroups against a prefill
// target, or the per-CU ticket sequences of §5.4.2).  Decode work is cut
// into one-wave units (§4.2.3 virtual decode CTAs).  Split partial results are merged by the
// last split to arrive, so no workgroup ever waits for another (the Silicon
// & Systems digest: results meet at synchronisation points and the
// scheduler must not deadlock).
//
// The result is exact softmax attention (the digest: fusion changes the
// order and placement of tiles, not the math); rounding aside, every path
// computes O = sum_j softmax_j(scale * q.K_j) V_j over the visible keys.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/pod_attn.h"
#include "pod_launch.h"
#include "pod_units.h"

namespace pod {

#define DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

struct Bf16 {
  static constexpr int bytes = 2;
};
struct F32 {
  static constexpr int bytes = 4;
};

constexpr float kNegInf = -__builtin_huge_valf();
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// The LDS a workgroup works in: four separately declared stage buffers (so
// the compiler can tell which one an LDS-DMA load writes and never has to
// wait for all of them before an LDS read) and the split's page ids.
struct LdsBufs {
  char* st[4];
  int* pids;
  int* flag;
};

// ------------------------------------------------------------------ helpers
DEV float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
DEV float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
// Round-to-nearest-even fp32 pair -> packed bf16 (v_cvt_pk_bf16_f32), a in bits 0..15.
DEV uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
DEV float safe_max(float m) { return m == kNegInf ? 0.0f : m; }

template <int CTRL>
DEV float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over each 16-lane row (DPP: swap pairs, swap pair-pairs, half-row mirror, row mirror).
DEV float row_sum16(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}
DEV float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }
// Reductions over lanes l and l ^ 16 (l ^ 32) with gfx950's row-swap
// permutes: swapping a register with itself hands every lane both values of
// its pair, with no LDS traffic and no lane-index register.
DEV float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEV float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
DEV float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
DEV float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
DEV int lane_id() { return __lane_id(); }
DEV int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Key of the compute unit this wave runs on: (XCC, shader engine, array, CU).
DEV uint32_t cu_key() {
  uint32_t hw = __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11));   // HW_REG_HW_ID
  uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)); // HW_REG_XCC_ID
  uint32_t cu = (hw >> 8) & 15u, sh = (hw >> 12) & 1u, se = (hw >> 13) & 7u;
  return ((xcc & 7u) << 8) | (se << 5) | (sh << 4) | cu;
}

template <int DW>
DEV void load_dw(uint32_t (&w)[DW], const void* ptr) {
  static_assert(DW == 2 || DW == 4 || DW == 8, "fragment width");
  if constexpr (DW == 2) {
    uint2 v = *reinterpret_cast<const uint2*>(ptr);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int i = 0; i < DW / 4; ++i) {
      uint4 v = reinterpret_cast<const uint4*>(ptr)[i];
      w[4 * i] = v.x;
      w[4 * i + 1] = v.y;
      w[4 * i + 2] = v.z;
      w[4 * i + 3] = v.w;
    }
  }
}

template <class E, int DW>
DEV void to_float(const uint32_t (&w)[DW], float* x) {
  if constexpr (E::bytes == 2) {
#pragma unroll
    for (int i = 0; i < DW; ++i) {
      x[2 * i] = bf16_lo(w[i]);
      x[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) x[i] = __uint_as_float(w[i]);
  }
}

// Partial dot product of two lane fragments (bf16: v_dot2_f32_bf16, exact products).
template <class E, int DW>
DEV float dot_frag(const uint32_t (&a)[DW], const uint32_t (&b)[DW]) {
  float acc = 0.0f;
  if constexpr (E::bytes == 2) {
#pragma unroll
    for (int i = 0; i < DW; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a[i]),
                                            __builtin_bit_cast(bf16x2_t, b[i]), acc, false);
  } else {
#pragma unroll
    for (int i = 0; i < DW; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  }
  return acc;
}

template <class E>
DEV void store_out(void* base, int64_t idx, float v) {
  if constexpr (E::bytes == 2) {
    reinterpret_cast<uint16_t*>(base)[idx] = (uint16_t)(pack_bf16(v, 0.0f) & 0xffffu);
  } else {
    reinterpret_cast<float*>(base)[idx] = v;
  }
}

// Split partials cross compute units on different XCDs, whose L2s are not
// coherent with each other.  They are written and read with device-scope
// accesses (cache policy sc1: written through to, and read from, the device
// coherence point), so publishing them needs no L2 writeback or invalidate:
// a wave waits until its device-scope stores have completed (vmcnt 0) and
// only then bumps the arrival counter, and the last arriver reads them back
// with device-scope loads after its counter update has returned.  The
// accesses go through buffer resources so that they can be 16 bytes wide.
constexpr int kDevScope = 16;        // buffer cache-policy bit sc1 (device scope)
constexpr int kNonTemporal = 2;      // buffer cache-policy bit nt (streamed once)
constexpr int kMergeLdsBytes = 2048; // wave-private LDS a merge needs for its weights

typedef __amdgpu_buffer_rsrc_t Rsrc;

// Buffer resource over `bytes` bytes from a wave-uniform base address.
DEV Rsrc dev_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                           (int)bytes, 0x00020000);
}
DEV void st_dev4(Rsrc r, uint32_t off, float a, float b, float c, float d) {
  const u32x4_t v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kDevScope);
}
DEV void st_dev1(Rsrc r, uint32_t off, float a) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a), r, (int)off, 0, kDevScope);
}
DEV f32x4_t ld_dev4(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kDevScope));
}
// Device-scope load from a per-lane address (global_load sc1).
DEV float ld_dev(const char* p) {
  return __hip_atomic_load(reinterpret_cast<float*>(const_cast<char*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory operation this wave issued has completed.
DEV void wait_vmem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt untouched
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Order this wave's LDS writes before its later LDS reads by other lanes.
DEV void wave_lds_sync() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Merge the S split partials of R output rows and store the rows.  The
// partial of split s is a block at part0 + s * sstride (bytes): acc [R][D]
// fp32 at +acc_off (rows contiguous), m (base 2) [R] at +m_off, l [R] at
// +l_off.  With M the largest m_s of a row, w_s = 2^(m_s - M), the row is
// sum_s w_s acc_s / sum_s w_s l_s; the sums run over the splits in index
// order, so the result does not depend on which split arrived last.  Output
// row i (i < nrows) goes to out0 + i * out_stride elements.  Up to IF
// 16-byte partial pieces per lane are loaded at once (more when a split's
// block is smaller).  `wl` is wave-private LDS of kMergeLdsBytes.
template <class E, int R, int D, int IF>
DEV void merge_rows(const char* part0, int64_t sstride, uint32_t acc_off, uint32_t m_off, uint32_t l_off,
                    int S, int nrows, char* out0, int64_t out_stride, float* wl) {
  static_assert(R <= 64 && 64 % R == 0, "rows per merge");
  constexpr int ITEMS = R * D / 4;                  // 16-byte pieces of one split's acc block
  constexpr int NL = (ITEMS + 63) / 64;             // pieces per lane
  constexpr int SC = kMergeLdsBytes / 4 / R;        // splits per chunk of LDS weights
  constexpr int SB = NL >= IF ? 1 : IF / NL;        // splits whose pieces are loaded together
  const uint32_t blk = (uint32_t)(l_off + R * 4 > acc_off + ITEMS * 16 ? l_off + R * 4 : acc_off + ITEMS * 16);
  const int lane = lane_id();
  const int rr = lane % R;
  auto split_rsrc = [&](int s) __attribute__((always_inline)) { return dev_rsrc(part0 + (int64_t)s * sstride, blk); };

  // (split, row) pairs q = s R + row, one per lane at a time: per-lane addresses
  float M = kNegInf;
  for (int q = lane; q < S * R; q += 64) M = fmaxf(M, ld_dev(part0 + (int64_t)(q / R) * sstride + m_off + 4 * rr));
#pragma unroll
  for (int o = R; o < 64; o <<= 1) M = fmaxf(M, xor_lane(M, o));
  M = safe_max(M);

  float L = 0.0f;
  f32x4_t acc[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) acc[j] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = 0; c0 < S; c0 += SC) {
    const int sc = min(SC, S - c0);
    for (int q = lane; q < sc * R; q += 64) {
      const char* ps = part0 + (int64_t)(c0 + q / R) * sstride;
      const float w = fast_exp2(ld_dev(ps + m_off + 4 * rr) - M);
      L += w * ld_dev(ps + l_off + 4 * rr);
      wl[q] = w;
    }
    wave_lds_sync();
    for (int s0 = 0; s0 < sc; s0 += SB) {
      f32x4_t v[SB][NL];
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const bool live = s0 + b < sc;
        const Rsrc rs = split_rsrc(c0 + s0 + (live ? b : 0));
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int it = j * 64 + lane;
          v[b][j] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f};
          if (live && (ITEMS % 64 == 0 || it < ITEMS)) v[b][j] = ld_dev4(rs, acc_off + 16 * it);
        }
      }
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        if (s0 + b >= sc) break;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
          const int row = (j * 64 + lane) * 4 / D;
          const float w = wl[(s0 + b) * R + (row < R ? row : 0)];
          acc[j] += w * v[b][j];
        }
      }
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int o = R; o < 64; o <<= 1) L += xor_lane(L, o);
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    const int it = j * 64 + lane;
    const int row = it * 4 / D, d = it * 4 % D;
    const float inv = 1.0f / __shfl(L, row < R ? row : 0, 64);
    if ((ITEMS % 64 == 0 || it < ITEMS) && row < nrows) {
      char* o = out0 + ((int64_t)row * out_stride + d) * E::bytes;
      const f32x4_t x = acc[j] * inv;
      if constexpr (E::bytes == 2) {
        uint2 w;
        w.x = pack_bf16(x[0], x[1]);
        w.y = pack_bf16(x[2], x[3]);
        *reinterpret_cast<uint2*>(o) = w;
      } else {
        *reinterpret_cast<float4*>(o) = make_float4(x[0], x[1], x[2], x[3]);
      }
    }
  }
}

// Count this wave's arrival after its partial stores completed; true for the
// last of `expected` arrivals.
DEV bool arrive_last(uint32_t* counter, uint32_t expected) {
  uint32_t old = 0;
  wait_vmem();
  if (lane_id() == 0) old = atomicAdd(counter, 1u);
  old = __shfl(old, 0, 64);
  return old == expected - 1;
}

// ---------------------------------------------------------- decode (a3, a4)
// One wave computes one (request r, kv head g, token split s) unit for the G
// query heads of g.  Lane layout: 4 token slots x 16 lanes; lane (slot, j)
// holds elements [j*D/16, (j+1)*D/16) of the tokens slot, slot+4, slot+8,
// slot+12 of each 16-token page, so a page is 4 coalesced row loads per
// operand and a dot product is a 16-lane DPP reduction.  Each slot keeps its
// own online softmax state; the four are combined at the end.
template <class E, int D>
struct DecFrag {
  static constexpr int EPL = D / 16;
  static constexpr int DW = EPL * E::bytes / 4;
};

// Find (request r, split s, splits S of r, base = splits of the requests
// before r) of decode unit `unit` (numbering and packing: pod_units.h) by a
// wave-wide prefix scan of the packed per-request counts, 64 requests at a
// time; `base + s` indexes the request's partial records.  Context lengths
// are clamped to the batch's largest host length, so a request never has
// more splits than the plan allowed for, and a unit whose records would
// fall outside the plan's (possible only if the device lengths differ from
// the host copy the launch was planned from) is dropped instead of written.
template <int RB>
DEV bool locate_unit(const PodParams& p, int unit, int& r, int& s, int& S, int& base) {
  const int lane = lane_id();
  const int ph = unit_phase_of(p.phase_start, unit_phases(p.tail_k, RB), unit);
  const uint32_t u = (uint32_t)(unit - p.phase_start[ph]);
  uint32_t key_acc = 0, base_acc = 0;
  for (int c0 = 0; c0 < p.N; c0 += kUnitScanLanes) {
    const int idx = c0 + lane;
    int L = idx < p.N ? min(p.ctx[idx], p.ctx_cap) : 0;
    L = max(L, 0);
    const uint32_t own = unit_pack(L, p.T, p.T2, p.tail_k, ph, RB);
    uint32_t incl = own;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off, 64);
      if (lane >= off) incl += v;
    }
    const uint32_t total = __shfl(incl, 63, 64);
    if (u < key_acc + unit_phase(total)) {
      const uint64_t hit = __ballot(key_acc + unit_phase(incl) > u);
      const int first = __builtin_ctzll(hit);
      r = c0 + first;
      unit_select(u, ph, key_acc, base_acc, __shfl(own, first, 64), __shfl(incl, first, 64), s, S, base);
      return base >= 0 && base + S <= p.d_units;
    }
    key_acc += unit_phase(total);
    base_acc += unit_total(total);
  }
  return false;
}

// Decode partial records: [G][D] acc, [G] m, [G] l, padded to 16 bytes.  The
// record of (request r, kv head g, split s) is g * units + base(r) + s, with
// base(r) the units of the requests before r, so the splits of one (r, g)
// are adjacent.
template <int D, int G>
struct DecRec {
  static constexpr int FLOATS = (G * (D + 2) + 3) & ~3;
  static constexpr uint32_t BYTES = FLOATS * 4;
  static constexpr uint32_t M_OFF = G * D * 4, L_OFF = G * D * 4 + G * 4;
};

template <int D, int G>
DEV Rsrc decode_record(const PodParams& p, int unit, int g) {
  return dev_rsrc(reinterpret_cast<const char*>(p.d_part) + ((int64_t)g * p.d_units + unit) * DecRec<D, G>::BYTES,
                  DecRec<D, G>::BYTES);
}

// Count this split's arrival at (r, g); the last of the S splits merges all
// partials of (r, g) in split order and restores the counter to zero.
// IF: 16-byte partial pieces per lane loaded at once (fewer in the
// 128-register envelope).
template <class E, int D, int G, int IF = (E::bytes == 2 ? 16 : 4)>
DEV void decode_finish(const PodParams& p, int r, int S, int base, int g, float* wl) {
  using Rc = DecRec<D, G>;
  uint32_t* cnt = p.d_cnt + (int64_t)r * p.hkv + g;
  if (!arrive_last(cnt, (uint32_t)S)) return;
  const char* part0 = reinterpret_cast<const char*>(p.d_part) + ((int64_t)g * p.d_units + base) * Rc::BYTES;
  char* out0 = reinterpret_cast<char*>(p.od) + ((int64_t)r * p.hq + (int64_t)g * G) * D * E::bytes;
  merge_rows<E, G, D, IF>(part0, Rc::BYTES, 0, Rc::M_OFF, Rc::L_OFF, S, G, out0, D, wl);
  if (lane_id() == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class E, int D, int G, int PF, int RB>
DEV void decode_wave(const PodParams& p, int wt, float* wl) {
  using Fr = DecFrag<E, D>;
  constexpr int EPL = Fr::EPL, DW = Fr::DW;
  const int lane = lane_id();
  const int hkv = p.hkv;
  const int g = wt % hkv;
  const int unit = wt / hkv;
  int r, s, S, base;
  if (!locate_unit<RB>(p, unit, r, s, S, base)) return;
  r = __builtin_amdgcn_readfirstlane(r);
  s = __builtin_amdgcn_readfirstlane(s);
  S = __builtin_amdgcn_readfirstlane(S);
  base = __builtin_amdgcn_readfirstlane(base);
  const int L = min(p.ctx[r], p.ctx_cap);
  int t0, t1;
  unit_range(L, p.T, p.T2, p.tail_k, s, t0, t1);
  const int npg = (t1 - t0 + kPageSize - 1) / kPageSize;
  const int slot = lane >> 4, j = lane & 15;

  // page ids of the split: lane i holds pages i, 64 + i, 128 + i, ...
  const int32_t* ptr = p.pt_d + (int64_t)r * p.stride + t0 / kPageSize;
  int pid[kSplitIdRegs];
#pragma unroll
  for (int k = 0; k < kSplitIdRegs; ++k) {
    int v = 0;
    if (64 * k + lane < npg) v = ptr[64 * k + lane];
    pid[k] = (int)min((uint32_t)v, p.num_pages - 1u);
  }
  auto page_id = [&](int i) __attribute__((always_inline)) {
    const int l = i & 63, k = i >> 6;
    int v = __builtin_amdgcn_readlane(pid[0], l);
#pragma unroll
    for (int j = 1; j < kSplitIdRegs; ++j)
      if (k == j) v = __builtin_amdgcn_readlane(pid[j], l);
    return v;
  };


  uint32_t q[G][DW];
  {
    const char* qb = reinterpret_cast<const char*>(p.qd) +
                     (((int64_t)r * p.hq + (int64_t)g * G) * D + j * EPL) * E::bytes;
#pragma unroll
    for (int h = 0; h < G; ++h) load_dw<DW>(q[h], qb + (int64_t)h * D * E::bytes);
  }
  const int64_t tok_bytes = (int64_t)hkv * D * E::bytes;
  const int64_t page_bytes = kPageSize * tok_bytes;
  const int64_t lane_off = ((int64_t)g * D + j * EPL) * E::bytes + slot * tok_bytes;
  const char* kb = reinterpret_cast<const char*>(p.k_pool) + lane_off;
  const char* vb = reinterpret_cast<const char*>(p.v_pool) + lane_off;

  float m[G], l[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.0f;
  }

  constexpr int NB = PF + 1;
  uint32_t kr[NB][4][DW], vr[NB][4][DW];

  auto issue = [&](uint32_t (&kd)[4][DW], uint32_t (&vd)[4][DW], int i) __attribute__((always_inline)) {
    const int64_t page = page_id(i);
    const int64_t off = page * page_bytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) load_dw<DW>(kd[u], kb + off + 4 * u * tok_bytes);
#pragma unroll
    for (int u = 0; u < 4; ++u) load_dw<DW>(vd[u], vb + off + 4 * u * tok_bytes);
  };

  auto consume = [&](const uint32_t (&kd)[4][DW], const uint32_t (&vd)[4][DW], int i) __attribute__((always_inline)) {
    const int tb = t0 + i * kPageSize + slot;
    float sc[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) sc[u][h] = row_sum16(dot_frag<E, DW>(q[h], kd[u]));
    bool valid[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) valid[u] = (tb + 4 * u) < t1;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sc[u][h] = valid[u] ? sc[u][h] * p.scale_log2 : kNegInf;
        mx = fmaxf(mx, sc[u][h]);
      }
      const float mnew = fmaxf(m[h], mx);
      const float mu = safe_max(mnew);
      const float alpha = fast_exp2(m[h] - mu);
      float ps = 0.0f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sc[u][h] = fast_exp2(sc[u][h] - mu);
        ps += sc[u][h];
      }
      l[h] = l[h] * alpha + ps;
      m[h] = mnew;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float v[EPL];
      to_float<E, DW>(vd[u], v);
#pragma unroll
      for (int e = 0; e < EPL; ++e) v[e] = valid[u] ? v[e] : 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(sc[u][h], v[e], acc[h][e]);
    }
  };

#pragma unroll
  for (int b = 0; b < PF; ++b)
    if (b < npg) issue(kr[b], vr[b], b);
  for (int i0 = 0; i0 < npg; i0 += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int i = i0 + b;
      if (i < npg) {
        if (i + PF < npg) issue(kr[(b + PF) % NB], vr[(b + PF) % NB], i + PF);
        consume(kr[b], vr[b], i);
      }
    }
  }

  // combine the four slots: common max, rescale, sum across rows of 16 lanes
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = fmaxf(m[h], xor_lane(m[h], 16));
    M = fmaxf(M, xor_lane(M, 32));
    const float f = fast_exp2(m[h] - safe_max(M));
    l[h] *= f;
    l[h] += xor_lane(l[h], 16);
    l[h] += xor_lane(l[h], 32);
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float a = acc[h][e] * f;
      a += xor_lane(a, 16);
      a += xor_lane(a, 32);
      acc[h][e] = a;
    }
    m[h] = M;
  }

  if (S == 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if ((h & 3) == slot) {
        const float inv = 1.0f / l[h];
        const int64_t o = ((int64_t)r * p.hq + (int64_t)g * G + h) * D + j * EPL;
#pragma unroll
        for (int e = 0; e < EPL; ++e) store_out<E>(p.od, o + e, acc[h][e] * inv);
      }
    }
    return;
  }

  // partial of this split
  using Rc = DecRec<D, G>;
  const Rsrc rs = decode_record<D, G>(p, base + s, g);
  static_assert(EPL % 4 == 0, "16-byte partial stores");
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if ((h & 3) == slot) {
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        st_dev4(rs, (h * D + j * EPL + e) * 4, acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      if (j == 0) {
        st_dev1(rs, Rc::M_OFF + h * 4, m[h]);
        st_dev1(rs, Rc::L_OFF + h * 4, l[h]);
      }
    }
  }
  decode_finish<E, D, G>(p, r, S, base, g, wl);
}

// bf16 decode on MFMA (v_mfma_f32_16x16x32_bf16), 16 query-head columns of
// which the G heads of kv head g are used.  Per pair of pages (32 keys):
//   S^T[key, head] = K Q^T     A = K rows (lane: key l%16, 8 d-elements at
//                              8*(l/16) of each 32-d chunk), B = Q^T in
//                              registers;
//   O^T[d, head] += V^T P^T    A = V^T via ds_read_b64_tr_b16 (the
//                              transposing LDS read), B = P^T straight from
//                              the S^T accumulators.
// K and V leave HBM in whole 256-byte head rows (16 lanes per token, four
// tokens per load, nontemporal), which streams far better than the 64-byte
// pieces the MFMA operand layout would ask for, and pass through this wave's
// own LDS buffer (no barrier: the buffer is private to the wave).  Row chunks
// are XOR-swizzled in LDS so the operand reads are free of bank conflicts.
// The key order inside an MFMA step is permuted identically on both sides
// (lane quad q feeds keys 4q..4q+3 of each page), so nothing is reshuffled.
// The softmax maximum is raised only when a score exceeds it by more than 8
// (base 2), so exp2(s - m) <= 256; the final division by l is unchanged, so
// the result is the same exact softmax.
template <int D>
struct DecMfma {
  static constexpr int KC = D / 32;          // QK k-chunks
  static constexpr int DB = D / 16;          // PV d-blocks
  static constexpr int ROWB = D * 2;         // bytes per token row of one head
  static constexpr int CHR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CHR;       // rows per load instruction
  static constexpr int NI = 16 / RPI;        // load instructions per page per operand
  static constexpr int OPB = 32 * ROWB;      // LDS bytes per operand (two pages)
  static constexpr int LDS_WAVE = 2 * OPB;   // K pages then V pages
  static constexpr float kLazy = 8.0f;
};


DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
// LDS chunk swizzles (measured on gfx950: 64 banks of 4 bytes, i.e. 256
// bytes per bank row; a ds_read_b128 is served 16 lanes per pass, a
// transposing ds_read_b64_tr_b16 32 lanes per pass).  Key rows of
// RB = 16 / CH rows (CH 16-byte chunks per row) share a bank row.
//  * K (both kernels): a b128 pass reads one logical chunk of 16 consecutive
//    rows, so XOR the chunk with the row's bank-row index over all chunk bits.
//  * V, prefill: a transposing pass reads 4 consecutive rows x 64 bytes, so
//    the rows' 64-byte groups are spread: XOR 4 (row / RB).
//  * V, decode: a transposing pass reads 8 consecutive rows x 32 bytes, so
//    the rows' 32-byte pairs are spread: XOR 2 (row / RB).
template <int CH>
DEV int ksw_rows(int row) { return (row / (16 / CH)) & (CH - 1); }
template <int CH>
DEV int vsw_prefill(int row) { return 4 * ((row / (16 / CH)) & (CH / 4 - 1)); }
template <int CH>
DEV int vsw_decode(int row) { return 2 * ((row / (16 / CH)) & (CH / 2 - 1)); }

template <int D, int G, int RB>
DEV void decode_wave_mfma(const PodParams& p, int wt, char* lds) {
  using C = DecMfma<D>;
  constexpr int KC = C::KC, DB = C::DB, NI = C::NI;
  const int lane = lane_id();
  const int hkv = p.hkv;
  const int g = wt % hkv;
  const int unit = wt / hkv;
  int r, s, S, base;
  if (!locate_unit<RB>(p, unit, r, s, S, base)) return;
  r = __builtin_amdgcn_readfirstlane(r);
  s = __builtin_amdgcn_readfirstlane(s);
  S = __builtin_amdgcn_readfirstlane(S);
  base = __builtin_amdgcn_readfirstlane(base);
  const int L = min(p.ctx[r], p.ctx_cap);
  int t0, t1;
  unit_range(L, p.T, p.T2, p.tail_k, s, t0, t1);
  const int npg = (t1 - t0 + kPageSize - 1) / kPageSize;
  const int npair = (npg + 1) >> 1;
  const int kk = lane & 15, q4 = lane >> 4;       // MFMA roles: key / head column, quad
  const int lrow = lane / C::CHR, lchk = lane % C::CHR;  // load role: row in group, chunk

  // page ids of the split: lane i holds pages i, 64 + i, 128 + i, ...
  const int32_t* ptr = p.pt_d + (int64_t)r * p.stride + t0 / kPageSize;
  int pid[kSplitIdRegs];
#pragma unroll
  for (int k = 0; k < kSplitIdRegs; ++k) {
    int v = 0;
    if (64 * k + lane < npg) v = ptr[64 * k + lane];
    pid[k] = (int)min((uint32_t)v, p.num_pages - 1u);
  }
  auto page_id = [&](int i) __attribute__((always_inline)) {
    // a select over the id registers (no branch: it sits between loads)
    const int l = i & 63, k = i >> 6;
    int v = __builtin_amdgcn_readlane(pid[0], l);
#pragma unroll
    for (int j = 1; j < kSplitIdRegs; ++j) {
      const int w = __builtin_amdgcn_readlane(pid[j], l);
      v = k == j ? w : v;
    }
    return v;
  };


  // Q^T operand: column = head kk (< G), rows d = 32c + 8q4 .. +8
  bf16x8_t qf[KC];
  {
    const char* qb = reinterpret_cast<const char*>(p.qd) +
                     (((int64_t)r * p.hq + (int64_t)g * G + kk) * D + 8 * q4) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < G) v = *reinterpret_cast<const uint4*>(qb + c * 64);
      qf[c] = as_bf16x8(v);
    }
  }
  // Loads are buffer loads on a descriptor of the page (a scalar base and a
  // 32-bit lane offset inside the page).  A page past the split's last gets
  // an empty descriptor: its loads return zeros without touching memory, so
  // every pair issues the same loads and the waits count them statically.
  const uint32_t tok_bytes = (uint32_t)hkv * D * 2;
  const uint32_t page_bytes = kPageSize * tok_bytes;
  const uint32_t lane_off = (uint32_t)lrow * tok_bytes + (uint32_t)g * C::ROWB + lchk * 16;
  char* kl = lds;            // K rows of the pair
  char* vl = lds + C::OPB;   // V rows of the pair

  f32x4_t acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.0f;

  u32x4_t kr[2][2][NI], vr[2][2][NI];
  // Keys past t1 (the rest of the last page, a missing second page) are
  // masked in compute(), so their values never reach the result.
  auto issue = [&](u32x4_t (&kd)[2][NI], u32x4_t (&vd)[2][NI], int pair) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const int pg = 2 * pair + pp;
      const int64_t off = (int64_t)page_id(min(pg, npg - 1)) * page_bytes;
      const int nrec = pg < npg ? (int)page_bytes : 0;
      const Rsrc rk = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(p.k_pool) + off), (short)0, nrec, 0x00020000);
      const Rsrc rv = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<char*>(reinterpret_cast<const char*>(p.v_pool) + off), (short)0, nrec, 0x00020000);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        kd[pp][u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(lane_off + u * C::RPI * tok_bytes), 0, kNonTemporal);
#pragma unroll
      for (int u = 0; u < NI; ++u)
        vd[pp][u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(lane_off + u * C::RPI * tok_bytes), 0, kNonTemporal);
    }
  };

  // K and V rows of a pair -> LDS; the registers are free for the next
  // loads once this is issued.  Only a pair that reaches past the split's
  // last key (uniform test) zeroes its invisible V rows.
  auto stage = [&](const u32x4_t (&kd)[2][NI], const u32x4_t (&vd)[2][NI], int pair) __attribute__((always_inline)) {
    const int kbase = t0 + 32 * pair;
    const bool full = kbase + 32 <= t1;
#pragma unroll
    for (int pp = 0; pp < 2; ++pp)
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        const int row = 16 * pp + u * C::RPI + lrow;
        *reinterpret_cast<u32x4_t*>(kl + row * C::ROWB + ((lchk ^ ksw_rows<C::CHR>(row)) << 4)) = kd[pp][u];
      }
    if (full) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int u = 0; u < NI; ++u) {
          const int row = 16 * pp + u * C::RPI + lrow;
          *reinterpret_cast<u32x4_t*>(vl + row * C::ROWB + ((lchk ^ vsw_decode<C::CHR>(row)) << 4)) = vd[pp][u];
        }
    } else {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int u = 0; u < NI; ++u) {
          const int row = 16 * pp + u * C::RPI + lrow;
          const bool ok = kbase + row < t1;
          *reinterpret_cast<u32x4_t*>(vl + row * C::ROWB + ((lchk ^ vsw_decode<C::CHR>(row)) << 4)) =
              ok ? vd[pp][u] : (u32x4_t){0u, 0u, 0u, 0u};
        }
    }
  };

  const float c2 = p.scale_log2;  // > 0, so the maximum commutes with the scaling
  auto compute = [&](int pair) __attribute__((always_inline)) {
    const int kbase = t0 + 32 * pair;
    const bool full = kbase + 32 <= t1;
    // S^T for both pages
    f32x4_t sc[2];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      sc[pp] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
      const int row = 16 * pp + kk;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kl + row * C::ROWB + (((4 * c + q4) ^ ksw_rows<C::CHR>(row)) << 4));
        sc[pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], sc[pp], 0, 0, 0);
      }
    }
    // raw scores (the scale goes into the exponent below); keys past t1
    // only in the split's last pair
    if (!full) {
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[pp][i] = kbase + 16 * pp + 4 * q4 + i < t1 ? sc[pp][i] : kNegInf;
    }
    float mloc = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mloc *= c2;
    if (__builtin_amdgcn_ballot_w64(mloc > m + C::kLazy) != 0) {
      float mm = fmaxf(mloc, xor_lane(mloc, 16));
      mm = fmaxf(mm, xor_lane(mm, 32));
      const float mnew = fmaxf(m, mm);
      const float alpha = fast_exp2(m - safe_max(mnew));
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] *= alpha;
      m = mnew;
    }
    const float nmu = -safe_max(m);
    // The row sum adds the same bf16 weights the PV product uses, so the
    // normalised weights sum to one: a dominant weight's rounding cancels
    // instead of scaling the whole output.
    uint32_t pw[4];
#pragma unroll
    for (int pp = 0; pp < 2; ++pp) {
      const float e0 = fast_exp2(fmaf(sc[pp][0], c2, nmu)), e1 = fast_exp2(fmaf(sc[pp][1], c2, nmu));
      const float e2 = fast_exp2(fmaf(sc[pp][2], c2, nmu)), e3 = fast_exp2(fmaf(sc[pp][3], c2, nmu));
      pw[2 * pp] = pack_bf16(e0, e1);
      pw[2 * pp + 1] = pack_bf16(e2, e3);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[2 * pp]), kOnes2, l, false);
      l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[2 * pp + 1]), kOnes2, l, false);
    }
    const bf16x8_t pf = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
    // O^T += V^T P^T; lane (quad q4, i = 4k + j) reads keys 4*q4 + k of each
    // page, d = 16b + 4j .. +4
    const int tk = (lane & 15) >> 2, tj = lane & 3;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const int chunk = 2 * b + (tj >> 1);
      const int r0 = 4 * q4 + tk, r1 = 16 + r0;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(
          vl + r0 * C::ROWB + ((chunk ^ vsw_decode<C::CHR>(r0)) << 4) + ((tj & 1) << 3)));
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(
          vl + r1 * C::ROWB + ((chunk ^ vsw_decode<C::CHR>(r1)) << 4) + ((tj & 1) << 3)));
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (short __attribute__((ext_vector_type(8)))){
          lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, acc[b], 0, 0, 0);
    }
  };

  // Two register buffers, both always in flight: a pair's registers are
  // reloaded with the pair after next as soon as they are staged in LDS,
  // before the pair is used, so the wave keeps two pairs (32 keys x K and V
  // each) of loads outstanding while it computes.  The scheduling barriers
  // keep the compiler from sinking the loads below the computation.
  // The loop runs an even number of pairs: a pair past the split's last has
  // every key masked and adds exact zeros, and its loads touch no memory.
  // With no branch inside, the loads of each buffer stay in issue order and
  // the compiler waits for exactly the pair it stages.
  issue(kr[0], vr[0], 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(kr[1], vr[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  for (int i = 0; i < npair; i += 2) {
    stage(kr[0], vr[0], i);
    issue(kr[0], vr[0], i + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute(i);
    stage(kr[1], vr[1], i + 1);
    issue(kr[1], vr[1], i + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(i + 1);
  }

  // l over the four key quads of each head column
  l += xor_lane(l, 16);
  l += xor_lane(l, 32);
  const int h = lane & 15;
  if (S == 1) {
    if (h < G) {
      const float inv = 1.0f / l;
      char* orow = reinterpret_cast<char*>(p.od) + (((int64_t)r * p.hq + (int64_t)g * G + h) * D + 4 * q4) * 2;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        uint2 w;
        w.x = pack_bf16(acc[b][0] * inv, acc[b][1] * inv);
        w.y = pack_bf16(acc[b][2] * inv, acc[b][3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * b) = w;
      }
    }
    return;
  }
  using Rc = DecRec<D, G>;
  const Rsrc rs = decode_record<D, G>(p, base + s, g);
  if (h < G) {
#pragma unroll
    for (int b = 0; b < DB; ++b) st_dev4(rs, (h * D + 16 * b + 4 * q4) * 4, acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    if (q4 == 0) {
      st_dev1(rs, Rc::M_OFF + h * 4, m);
      st_dev1(rs, Rc::L_OFF + h * 4, l);
    }
  }
  decode_finish<Bf16, D, G>(p, r, S, base, g, reinterpret_cast<float*>(lds));
}

// bf16 decode wave of the four-workgroups-per-CU envelope (at most 128
// registers per lane, 8 KB of LDS per wave): one page (16 keys) per step
// through the wave's LDS buffer (K rows then V rows).  The next page's loads
// are issued as soon as the current page is in LDS, so one page per wave is
// in flight while the current one is computed, and the registers hold one
// page of loads instead of two pairs.  QK^T on v_mfma_f32_16x16x32_bf16 as
// in decode_wave_mfma; PV on v_mfma_f32_16x16x16_bf16 with the page's 16
// keys as the k dimension (one transposing read per 16-wide d tile).
template <int D>
struct DecMfma4 {
  static constexpr int KC = D / 32;          // QK k-chunks
  static constexpr int DB = D / 16;          // PV d-blocks
  static constexpr int ROWB = D * 2;         // bytes per token row of one head
  static constexpr int CHR = D / 8;          // 16-byte chunks per row
  static constexpr int RPI = 64 / CHR;       // rows per load instruction
  static constexpr int NI = 16 / RPI;        // load instructions per page per operand
  static constexpr int OPB = 16 * ROWB;      // LDS bytes per operand (one page)
  static constexpr int LDS_WAVE = 2 * OPB;   // K page then V page
  static constexpr float kLazy = 8.0f;
};

template <int D, int G, int RB>
DEV void decode_wave_mfma4(const PodParams& p, int wt, char* lds, int* wpids) {
  using C = DecMfma4<D>;
  constexpr int KC = C::KC, DB = C::DB, NI = C::NI;
  const int lane = lane_id();
  const int hkv = p.hkv;
  const int g = wt % hkv;
  const int unit = wt / hkv;
  int r, s, S, base;
  if (!locate_unit<RB>(p, unit, r, s, S, base)) return;
  r = __builtin_amdgcn_readfirstlane(r);
  s = __builtin_amdgcn_readfirstlane(s);
  S = __builtin_amdgcn_readfirstlane(S);
  base = __builtin_amdgcn_readfirstlane(base);
  const int L = min(p.ctx[r], p.ctx_cap);
  int t0, t1;
  unit_range(L, p.T, p.T2, p.tail_k, s, t0, t1);
  const int npg = (t1 - t0 + kPageSize - 1) / kPageSize;
  const int kk = lane & 15, q4 = lane >> 4;       // MFMA roles: key / head column, quad
  const int lrow = lane / C::CHR, lchk = lane % C::CHR;  // load role: row in group, chunk

  // page ids of the split in the wave's LDS slice (at most 256 of them):
  // registers are too scarce in this envelope to hold them.  LDS operations
  // of a wave run in order, so later reads see these writes.
  const int32_t* ptr = p.pt_d + (int64_t)r * p.stride + t0 / kPageSize;
#pragma unroll
  for (int k = 0; k < kSplitIdRegs; ++k)
    if (64 * k + lane < npg) wpids[64 * k + lane] = (int)min((uint32_t)ptr[64 * k + lane], p.num_pages - 1u);
  auto page_id = [&](int i) __attribute__((always_inline)) { return wpids[min(i, npg - 1)]; };

  // Q^T operand: column = head kk (< G), rows d = 32c + 8q4 .. +8
  bf16x8_t qf[KC];
  {
    const char* qb = reinterpret_cast<const char*>(p.qd) +
                     (((int64_t)r * p.hq + (int64_t)g * G + kk) * D + 8 * q4) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kk < G) v = *reinterpret_cast<const uint4*>(qb + c * 64);
      qf[c] = as_bf16x8(v);
    }
  }
  // Loads are buffer loads on a descriptor of the page (a scalar base and a
  // 32-bit lane offset inside the page), so no 64-bit lane pointers occupy
  // registers.
  const uint32_t tok_bytes = (uint32_t)hkv * D * 2;
  const uint32_t page_bytes = kPageSize * tok_bytes;
  const uint32_t lane_off = (uint32_t)lrow * tok_bytes + (uint32_t)g * C::ROWB + lchk * 16;
  char* kl = lds;            // K rows of the page
  char* vl = lds + C::OPB;   // V rows of the page

  f32x4_t acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.0f;

  u32x4_t kr[NI], vr[NI];
  auto issue = [&](int pid) __attribute__((always_inline)) {
    const int64_t off = (int64_t)__builtin_amdgcn_readfirstlane(pid) * page_bytes;
    const Rsrc rk = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.k_pool) + off), (short)0, (int)page_bytes, 0x00020000);
    const Rsrc rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.v_pool) + off), (short)0, (int)page_bytes, 0x00020000);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      kr[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(lane_off + u * C::RPI * tok_bytes), 0, kNonTemporal);
#pragma unroll
    for (int u = 0; u < NI; ++u)
      vr[u] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(lane_off + u * C::RPI * tok_bytes), 0, kNonTemporal);
  };
  const int tk = (lane & 15) >> 2, tj = lane & 3;
  const int vr0 = 4 * q4 + tk;  // the key row this lane feeds to the transposing reads

  issue(page_id(0));
  int pid_next = page_id(1);
  for (int i = 0; i < npg; ++i) {
    const int pid_after = page_id(i + 2);  // read a page ahead of its use
    const int kbase = t0 + kPageSize * i;
    // page i -> LDS; LDS operations of a wave run in order, so these writes
    // land after the previous page's reads.  Only a split's last page can
    // hold invisible rows; their V rows are zeroed (a uniform branch, so no
    // copies of the loaded rows are kept).
    if (kbase + kPageSize > t1) {
#pragma unroll
      for (int u = 0; u < NI; ++u)
        if (kbase + u * C::RPI + lrow >= t1) vr[u] = (u32x4_t){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      const int row = u * C::RPI + lrow;
      *reinterpret_cast<u32x4_t*>(kl + row * C::ROWB + ((lchk ^ ksw_rows<C::CHR>(row)) << 4)) = kr[u];
      *reinterpret_cast<u32x4_t*>(vl + row * C::ROWB + ((lchk ^ vsw_decode<C::CHR>(row)) << 4)) = vr[u];
    }
    // S^T of the page
    f32x4_t sc = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kl + kk * C::ROWB + (((4 * c + q4) ^ ksw_rows<C::CHR>(kk)) << 4));
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[c], sc, 0, 0, 0);
    }
    // the next page's loads fly during the softmax and PV of this one (issued
    // after the K reads so that both sets of operands are never live at once)
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < npg) issue(pid_next);
    pid_next = pid_after;
    float mloc = kNegInf;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = kbase + 4 * q4 + j < t1;
      const float v = ok ? sc[j] * p.scale_log2 : kNegInf;
      sc[j] = v;
      mloc = fmaxf(mloc, v);
    }
    if (__builtin_amdgcn_ballot_w64(mloc > m + C::kLazy) != 0) {
      const float mm = max_xor32(max_xor16(mloc));
      const float mnew = fmaxf(m, mm);
      const float alpha = fast_exp2(m - safe_max(mnew));
      l *= alpha;
#pragma unroll
      for (int b = 0; b < DB; ++b) acc[b] *= alpha;
      m = mnew;
    }
    const float mu = safe_max(m);
    // the row sum adds the bf16 weights the PV product uses
    uint32_t pw[2];
    pw[0] = pack_bf16(fast_exp2(sc[0] - mu), fast_exp2(sc[1] - mu));
    pw[1] = pack_bf16(fast_exp2(sc[2] - mu), fast_exp2(sc[3] - mu));
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[0]), kOnes2, l, false);
    l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[1]), kOnes2, l, false);
    const i16x4_t pf = __builtin_bit_cast(i16x4_t, make_uint2(pw[0], pw[1]));
    // O^T += V^T P^T: lane (quad q4, 4k + j) reads key 4 q4 + k, d = 16b + 4j .. +4;
    // four d blocks' operands in registers at a time
#pragma unroll
    for (int b0 = 0; b0 < DB; b0 += 4) {
      i16x4_t va[4];
#pragma unroll
      for (int e = 0; e < 4 && b0 + e < DB; ++e) {
        const int chunk = 2 * (b0 + e) + (tj >> 1);
        va[e] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(
            vl + vr0 * C::ROWB + ((chunk ^ vsw_decode<C::CHR>(vr0)) << 4) + ((tj & 1) << 3)));
      }
#pragma unroll
      for (int e = 0; e < 4 && b0 + e < DB; ++e)
        acc[b0 + e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[e], pf, acc[b0 + e], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // l over the four key quads of each head column
  l = sum_xor32(sum_xor16(l));
  const int h = lane & 15;
  if (S == 1) {
    if (h < G) {
      const float inv = 1.0f / l;
      char* orow = reinterpret_cast<char*>(p.od) + (((int64_t)r * p.hq + (int64_t)g * G + h) * D + 4 * q4) * 2;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        uint2 w;
        w.x = pack_bf16(acc[b][0] * inv, acc[b][1] * inv);
        w.y = pack_bf16(acc[b][2] * inv, acc[b][3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * b) = w;
      }
    }
    return;
  }
  using Rc = DecRec<D, G>;
  const Rsrc rs = decode_record<D, G>(p, base + s, g);
  if (h < G) {
#pragma unroll
    for (int b = 0; b < DB; ++b) st_dev4(rs, (h * D + 16 * b + 4 * q4) * 4, acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    if (q4 == 0) {
      st_dev1(rs, Rc::M_OFF + h * 4, m);
      st_dev1(rs, Rc::L_OFF + h * 4, l);
    }
  }
  decode_finish<Bf16, D, G, 4>(p, r, S, base, g, reinterpret_cast<float*>(lds));
}

// RB: remainder phases of the unit numbering (1 in fused launches,
// kRemBuckets in decode-only launches; the plan numbers the units alike)
template <int D, int G, int RB = 1>
DEV void decode_wg4(const PodParams& p, int wg_task, const LdsBufs& lb) {
  const int wt = wg_task * kWavesPerWG + wave_id();
  if (wt >= p.d_wave_tasks) return;
  const int w = wave_id();
  char* buf = w == 0 ? lb.st[0] : w == 1 ? lb.st[1] : w == 2 ? lb.st[2] : lb.st[3];
  decode_wave_mfma4<D, G, RB>(p, wt, buf, lb.pids + w * (kSplitIdRegs * 64));
}

template <class E, int D, int G, int PF, int RB = 1>
DEV void decode_wg(const PodParams& p, int wg_task, const LdsBufs& lb) {
  const int wt = wg_task * kWavesPerWG + wave_id();
  if (wt >= p.d_wave_tasks) return;
  const int w = wave_id();
  char* buf = w == 0 ? lb.st[0] : w == 1 ? lb.st[1] : w == 2 ? lb.st[2] : lb.st[3];
  if constexpr (E::bytes == 2)
    decode_wave_mfma<D, G, RB>(p, wt, buf);
  else
    decode_wave<E, D, G, PF, RB>(p, wt, reinterpret_cast<float*>(buf));
}

// ---------------------------------------------------------- prefill (a2, a4)
// A prefill task is (chunk, tile, KV split).  A tile is (row block, kv head
// g, head group): 4 waves, wave w takes 32 (bf16) or 64 (fp32) consecutive
// chunk rows of one query head of g.  K/V blocks of the split's key range
// are staged once in LDS and shared by the 4 waves (the GQA heads of one kv
// head reuse the same keys).  Rows are chunk-local: row i of the chunk sits
// at absolute position P0 + i and at row row_base + i of the packed q and o.
struct TaskGeom {
  int C, P0, Lp;      // the chunk: rows, offset, keys
  int splits, tiles;  // the chunk's splits per tile and tiles
  int row_base;       // the chunk's first row in q and o
  const int32_t* pt;  // the chunk's page table
  int tile, split, rb, g, hg;
  int head, row0;     // this wave's head and first row
  int k0, k1;         // split key range, clipped to the tile's causal end
  int kw;             // this wave's last visible key + 1 within the split
};

typedef __attribute__((address_space(4))) const char karg_char_t;
typedef __attribute__((address_space(4))) const PfChunk karg_chunk_t;

// Chunk c of the launch, read from the kernel-argument segment with a
// uniform index (a scalar load; indexing the by-value parameter would copy
// the table to scratch).  The parameter block is the kernels' only argument.
DEV PfChunk load_chunk(int c) {
  karg_chunk_t* t =
      (karg_chunk_t*)((karg_char_t*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(PodParams, ch)) + c;
  PfChunk r;
  r.task_base = t->task_base;
  r.tile_base = t->tile_base;
  r.row_base = t->row_base;
  r.pt_base = t->pt_base;
  r.C = t->C;
  r.P0 = t->P0;
  r.splits = t->splits;
  r.split_keys = t->split_keys;
  r.row_blocks = t->row_blocks;
  return r;
}

DEV int chunk_task_base(int c) {
  return ((karg_chunk_t*)((karg_char_t*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(PodParams, ch)) + c)
      ->task_base;
}

template <int RPW>
DEV TaskGeom prefill_geom(const PodParams& p, int task) {
  TaskGeom t;
  task = __builtin_amdgcn_readfirstlane(task);
  // the last chunk whose first task is <= task (binary search, scalar loads)
  int lo = 0, hi = p.n_chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (task >= chunk_task_base(mid))
      lo = mid;
    else
      hi = mid - 1;
  }
  const PfChunk ch = load_chunk(lo);
  t.C = ch.C;
  t.P0 = ch.P0;
  t.Lp = ch.C + ch.P0;
  t.splits = ch.splits;
  t.tiles = ch.row_blocks * p.head_groups * p.hkv;
  t.row_base = ch.row_base;
  t.pt = p.pt_p + ch.pt_base;
  int i = task - ch.task_base;
  t.g = i % p.hkv;
  i /= p.hkv;
  t.hg = i % p.head_groups;
  i /= p.head_groups;
  const int rbi = i % ch.row_blocks;
  t.split = i / ch.row_blocks;
  t.rb = ch.row_blocks - 1 - rbi;  // longest (latest) row blocks first
  t.tile = ch.tile_base + (t.rb * p.head_groups + t.hg) * p.hkv + t.g;
  const int w = wave_id();
  const int G = p.hq / p.hkv;
  t.head = t.g * G + t.hg * p.heads_per_tile + (w % p.heads_per_tile);
  t.row0 = t.rb * p.rows_per_tile + (w / p.heads_per_tile) * RPW;
  const int tile_end = t.P0 + min(t.C, (t.rb + 1) * p.rows_per_tile);  // causal end of the tile
  t.k0 = t.split * ch.split_keys;
  t.k1 = min(t.k0 + ch.split_keys, tile_end);
  t.kw = min(t.k1, t.P0 + min(t.C, t.row0 + RPW));
  return t;
}

// Copy the physical ids of pages [pg0, pg0 + n) of a page table into LDS
// (clamped into the pool).
DEV void preload_page_ids(const int32_t* pt, uint32_t num_pages, int pg0, int n, int* pids) {
  for (int i = threadIdx.x; i < n; i += 256) pids[i] = (int)min((uint32_t)pt[pg0 + i], num_pages - 1u);
}

// Wait until at most N of this wave's vector memory operations are in flight
// and all its LDS operations are done (s_waitcnt vmcnt(N) lgkmcnt(0)).
template <int N>
DEV void wait_vm_lgkm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

typedef __attribute__((address_space(3))) void lds_void_t;


// bf16 prefill tile: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_bf16.
// Lane l owns query row (l & 31) of its wave; its half h = l >> 5 owns half of
// every 32-key score column, so row max and row sum are mostly in-lane.
//
// K/V blocks of 32 keys stream from the paged pool straight into LDS
// (global_load_lds_dwordx4, no register staging) through NS stages, NS - 1
// blocks ahead of the block being computed.  Rows are stored unpadded; the
// 16-byte chunks of each row are XOR-swizzled on the global side so that the
// MFMA operand reads hit distinct LDS banks: K row r keeps chunk c at
// c ^ (r & 7) (read 32 rows x 16 bytes with ds_read_b128), V row r at
// c ^ 2(r & 3) (read 4 rows x 32 bytes per 16 lanes with the transposing
// ds_read_b64_tr_b16, which hands each lane one d-column of 4 keys).
template <int D>
struct PfBf16 {
  static constexpr int RPW = 32;                 // query rows per wave
  static constexpr int BN = 32;                  // keys per staged block
  static constexpr int NS = 4;                   // LDS stages
  static constexpr int ROWB = D * 2;             // bytes per key row
  static constexpr int OPB = BN * ROWB;          // bytes per operand per stage
  static constexpr int STAGE = 2 * OPB;          // K block then V block
  static constexpr int CH = D / 8;               // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;            // rows per 64-lane DMA instruction
  static constexpr int IPW = BN / RPI / kWavesPerWG;  // DMA instructions per operand per wave
  static constexpr int LPB = 2 * IPW;            // DMA loads per wave per block
  static constexpr int PIDS = kMaxSplitKeys / kPageSize;
  static constexpr int LDS = NS * STAGE + PIDS * 4;
  static_assert(IPW >= 1, "block too small for the workgroup");
};

// Per-lane byte offsets (within a page) of a wave's K and V DMA loads: load
// i of the wave fetches 16-byte chunk pos ^ swizzle(row) of token slot row &
// 15 into LDS row `row` of the block.  Blocks start on page boundaries, so
// the offsets are the same for every block that lies inside the request.
template <int D>
struct PfDma {
  static constexpr int IPW = PfBf16<D>::IPW;
  uint32_t k[IPW], v[IPW];
};

// V rows are swizzled for the PV operand reads of the tile that consumes
// them: the 32-row tile reads 4 rows x 64 bytes per transposing pass
// (vsw_prefill), the 16-row tile 8 rows x 32 bytes (vsw_decode).
template <int CH, bool V16>
DEV int vsw_tile(int row) { return V16 ? vsw_decode<CH>(row) : vsw_prefill<CH>(row); }

template <int D, bool V16 = false>
DEV PfDma<D> prefill_dma_offsets(int64_t tok_bytes) {
  using C = PfBf16<D>;
  const int lane = lane_id();
  const int pos = lane % C::CH, lrow = lane / C::CH;
  PfDma<D> o;
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int row = (wave_id() * C::IPW + i) * C::RPI + lrow;
    o.k[i] = (uint32_t)((row & 15) * tok_bytes) + ((pos ^ ksw_rows<C::CH>(row)) << 4);
    o.v[i] = (uint32_t)((row & 15) * tok_bytes) + ((pos ^ vsw_tile<C::CH, V16>(row)) << 4);
  }
  return o;
}

// Page of the keys this wave loads for the block at kb0: a wave's loads
// cover consecutive rows inside one page.  Rows past the request re-read its
// last key (never a NaN tail slot); they are masked later.
template <int D>
DEV int prefill_wave_page_index(int kb0, int Lp, int pg0) {
  using C = PfBf16<D>;
  static_assert(C::IPW * C::RPI <= kPageSize, "a wave's rows must stay in one page");
  return (min(kb0 + wave_id() * C::IPW * C::RPI, Lp - 1) >> 4) - pg0;
}

// Issue the DMA loads of the block at kb0 (page id `page` for this wave).
template <int D, bool V16 = false>
DEV void prefill_issue_block(const char* kpool, const char* vpool, int64_t tok_bytes, int page, int Lp, int kb0,
                             const PfDma<D>& off, char* stage) {
  using C = PfBf16<D>;
  const char* kp = kpool + (int64_t)page * kPageSize * tok_bytes;
  const char* vp = vpool + (int64_t)page * kPageSize * tok_bytes;
  const bool tail = kb0 + C::BN > Lp;  // the block reaches past the request's last key
  const int lane = lane_id();
  const int pos = lane % C::CH, lrow = lane / C::CH;
  // The DMA instructions stay outside any branch: only the offsets differ
  // for a tail block, so the compiler keeps its per-buffer wait tracking.
  // They are buffer loads on a descriptor of the page: with the global form
  // the compiler turns every later LDS wait of the wave into a full
  // lgkmcnt(0) while a DMA is in flight (the prefill ran 3-4% slower).
  const Rsrc rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kp), (short)0, kPageSize * (int)tok_bytes, 0x00020000);
  const Rsrc rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vp), (short)0, kPageSize * (int)tok_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < C::IPW; ++i) {
    const int ins = wave_id() * C::IPW + i;
    uint32_t ko = off.k[i], vo = off.v[i];
    if (tail) {
      const int row = ins * C::RPI + lrow;
      const uint32_t slot = (uint32_t)(min(kb0 + row, Lp - 1) & 15) * (uint32_t)tok_bytes;
      ko = slot + ((pos ^ ksw_rows<C::CH>(row)) << 4);
      vo = slot + ((pos ^ vsw_tile<C::CH, V16>(row)) << 4);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(stage + ins * 1024), 16, ko, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(stage + C::OPB + ins * 1024), 16, vo, 0, 0, 0);
  }
}

// Prefill partial of one task (tile, split): acc [RH][D] fp32, m [RH], l [RH]
// for the tile's RH = 4 * RPW row-heads, wave w owning rows [w RPW, (w+1) RPW).
template <int D, int RPW>
struct PfRec {
  static constexpr int RH = RPW * kWavesPerWG;
  static constexpr uint32_t BYTES = RH * (D + 2) * 4;
  static DEV uint32_t acc_off(int w) { return (uint32_t)(w * RPW * D * 4); }
  static DEV uint32_t m_off(int w) { return (uint32_t)(RH * D * 4 + w * RPW * 4); }
  static DEV uint32_t l_off(int w) { return (uint32_t)(RH * (D + 1) * 4 + w * RPW * 4); }
};


// Tile-level arrival and merge, shared by both prefill flavours: every
// thread waits for its own partial stores, the workgroup synchronises, one
// thread counts the arrival, and the last split's workgroup merges.
template <class E, int D, int RPW>
DEV void prefill_finish_split(const PodParams& p, const TaskGeom& t, int task, const LdsBufs& lb) {
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) *lb.flag = atomicAdd(p.p_cnt + t.tile, 1u) == (uint32_t)t.splits - 1u;
  __syncthreads();
  if (!*lb.flag) return;
  const int w = wave_id();
  using Rc = PfRec<D, RPW>;
  // Tasks of one tile differ only in their split: task = split * tiles + (tile
  // position), so split s of this tile is task - (split - s) * tiles.
  const char* part0 = reinterpret_cast<const char*>(p.p_part) + (int64_t)(task - t.split * t.tiles) * Rc::BYTES;
  char* out0 = reinterpret_cast<char*>(p.op) + ((int64_t)(t.row_base + t.row0) * p.hq + t.head) * D * E::bytes;
  float* wl = reinterpret_cast<float*>(w == 0 ? lb.st[0] : w == 1 ? lb.st[1] : w == 2 ? lb.st[2] : lb.st[3]);
  merge_rows<E, RPW, D, (RPW == 16 ? 4 : 16)>(part0, (int64_t)t.tiles * Rc::BYTES, Rc::acc_off(w), Rc::m_off(w), Rc::l_off(w), t.splits,
                        min(RPW, t.C - t.row0), out0, (int64_t)p.hq * D, wl);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_store(p.p_cnt + t.tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
DEV void prefill_tile_bf16(const PodParams& p, int task, const LdsBufs& lb) {
  using C = PfBf16<D>;
  static_assert(C::NS == 4, "the block loop is unrolled over four stage buffers");
  constexpr int KS = D / 16;   // MFMA k-steps over d
  constexpr int DB = D / 32;   // 32-wide d blocks of O^T
  const TaskGeom t = prefill_geom<C::RPW>(p, task);
  const int lane = lane_id();
  const int half = lane >> 5, rl = lane & 31;
  const int row = t.row0 + rl;
  const int64_t tok_bytes = (int64_t)p.hkv * D * 2;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)t.g * D * 2;
  const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)t.g * D * 2;

  // Q^T operand: lane holds d = 16 ks + 8 half .. +8 of its row
  bf16x8_t qf[KS];
  {
    const char* qrow =
        reinterpret_cast<const char*>(p.qp) + (((int64_t)(t.row_base + row) * p.hq + t.head) * D + 8 * half) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < t.C) v = *reinterpret_cast<const uint4*>(qrow + ks * 32);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.0f;
  float m = kNegInf, l = 0.0f;

  const int nblk = t.k1 > t.k0 ? (t.k1 - t.k0 + C::BN - 1) / C::BN : 0;
  const int lim = t.P0 + row;  // last visible key of this lane's row

  int* pids = lb.pids;
  const int pg0 = t.k0 / kPageSize;
  const int pg1 = min((t.Lp + kPageSize - 1) / kPageSize, (t.k0 + nblk * C::BN + kPageSize - 1) / kPageSize);
  preload_page_ids(t.pt, p.num_pages, pg0, pg1 - pg0, pids);
  __syncthreads();

  if (nblk > 0) {
    const PfDma<D> dma = prefill_dma_offsets<D>(tok_bytes);
    auto kb_of = [&](int b) __attribute__((always_inline)) { return t.k0 + min(b, nblk - 1) * C::BN; };
    // prologue: blocks 0 .. NS-2 (past the last block, the last block again)
#pragma unroll
    for (int s = 0; s < C::NS - 1; ++s)
      prefill_issue_block<D>(kpool, vpool, tok_bytes,
                             __builtin_amdgcn_readfirstlane(pids[prefill_wave_page_index<D>(kb_of(s), t.Lp, pg0)]),
                             t.Lp, kb_of(s), dma, lb.st[s]);
    // page id of the next block to issue, read one step ahead of its use
    int pid_next = pids[prefill_wave_page_index<D>(kb_of(C::NS - 1), t.Lp, pg0)];
    // Per-lane byte offsets of the K operand reads inside a stage.  The mask
    // (a no-op: they are below one stage) tells the compiler they are
    // non-negative, so the stage base folds into the LDS read's immediate
    // offset instead of costing an add per read.
    uint32_t koff[KS];
    {
      const int ksw = ksw_rows<C::CH>(rl);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        koff[ks] = (uint32_t)(rl * C::ROWB + (((2 * ks + half) ^ ksw) << 4)) & 0xffffu;
    }
    const int gq = lane >> 4, ti = lane & 15;
    const int th = gq >> 1, tdh = gq & 1, tk = ti >> 2, tj = ti & 3;
    const float c2 = p.scale_log2;

    // S^T (32 keys x 32 rows) of the block in stage `st`, unscaled
    auto qk = [&](const char* st) __attribute__((always_inline)) {
      f32x16_t s;
#pragma unroll
      for (int j = 0; j < 16; ++j) s[j] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(st + koff[ks]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
      }
      return s;
    };
    // Online softmax of one block (base 2; the running max is raised only when
    // a scaled score exceeds it by more than 8), in two parts.  The first
    // holds the rare branches: the causal mask of a diagonal block and the
    // rescale of o and l; it returns -max.
    auto softmax_max = [&](f32x16_t& sc, int kb0) __attribute__((always_inline)) {
      if ((kb0 + C::BN - 1) > (t.P0 + t.row0)) {  // diagonal block: causal mask
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = kb0 + 8 * (j >> 2) + 4 * half + (j & 3);
          sc[j] = key <= lim ? sc[j] : kNegInf;
        }
      }
      float mx = sc[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mx = fmaxf(mx, sc[j]);
      mx *= c2;  // this lane's half of the row; scale > 0: the max commutes with it
      // A row's maximum exceeds m + 8 only if one of its two halves does, so
      // the halves (lanes l and l ^ 32) are combined on the rare rescale path
      // only, keeping the cross-lane exchange off every block's critical path.
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
        const float mnew = fmaxf(m, fmaxf(mx, xor_lane(mx, 32)));
        const float alpha = fast_exp2(m - safe_max(mnew));
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        m = mnew;
      }
      return -safe_max(m);
    };
    // The second part is straight-line code: the weights of this block (vector
    // unit), the QK of the next block (matrix cores, independent of the
    // weights) and O^T += V^T P^T, so the scheduler can interleave them.
    auto weights_qk_pv = [&](const f32x16_t& sc, float nmu, const char* st, f32x16_t& sn, const char* st_next)
        __attribute__((always_inline)) {
      bf16x8_t pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint32_t w4[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          const float e0 = fast_exp2(fmaf(sc[8 * ks + 2 * q2], c2, nmu));
          const float e1 = fast_exp2(fmaf(sc[8 * ks + 2 * q2 + 1], c2, nmu));
          w4[q2] = pack_bf16(e0, e1);
          // l sums the bf16 weights the PV product uses, so they normalise exactly
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w4[q2]), kOnes2, l, false);
        }
        pf[ks] = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
      }
      sn = qk(st_next);
      // keys 16ks + 4th + tk (first transposing read) and + 8 (second)
      const char* vt = st + C::OPB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int c = 4 * db + 2 * tdh + (tj >> 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 16 * ks + 4 * th + tk, r1 = r0 + 8;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + r0 * C::ROWB + ((c ^ vsw_prefill<C::CH>(r0)) << 4) + ((tj & 1) << 3)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vt + r1 * C::ROWB + ((c ^ vsw_prefill<C::CH>(r1)) << 4) + ((tj & 1) << 3)));
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, (short __attribute__((ext_vector_type(8)))){
              lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ks], o[db], 0, 0, 0);
        }
      }
    };

    // block 0 must be in LDS before the first QK: blocks 1 and 2 may still fly
    wait_vm_lgkm<C::LPB * (C::NS - 2)>();
    __builtin_amdgcn_s_barrier();
    // Scores of even blocks live in s_even, of odd blocks in s_odd (NS is even).
    f32x16_t s_even = qk(lb.st[0]), s_odd;
    // Step b: QK of block b+1 is issued ahead of the softmax and PV of block
    // b, so the matrix cores work while the vector unit does the softmax.
    // Steps past nblk keep the same DMA/barrier sequence (re-loading the last
    // block) so every stage buffer sees one straight-line wait pattern.
    for (int b0 = 0; b0 < nblk; b0 += C::NS) {
#pragma unroll
      for (int u = 0; u < C::NS; ++u) {
        const int b = b0 + u;
        // block b+1 has landed once at most one newer block is in flight
        wait_vm_lgkm<C::LPB * (C::NS - 3)>();
        __builtin_amdgcn_s_barrier();
        const int page = __builtin_amdgcn_readfirstlane(pid_next);
        prefill_issue_block<D>(kpool, vpool, tok_bytes, page, t.Lp, kb_of(b + C::NS - 1), dma,
                               lb.st[(u + C::NS - 1) % C::NS]);
        pid_next = pids[prefill_wave_page_index<D>(kb_of(b + C::NS), t.Lp, pg0)];
        // Blocks past the wave's causal end are fully masked (weights 0), and
        // the QK past the last block reads a stage that holds the last block
        // again and is never used, so the body needs no further branches.
        if (b < nblk) {
          const int kb0 = t.k0 + b * C::BN;
          if (u % 2 == 0) {
            const float nmu = softmax_max(s_even, kb0);
            weights_qk_pv(s_even, nmu, lb.st[u], s_odd, lb.st[(u + 1) % C::NS]);
          } else {
            const float nmu = softmax_max(s_odd, kb0);
            weights_qk_pv(s_odd, nmu, lb.st[u], s_even, lb.st[(u + 1) % C::NS]);
          }
        }
      }
    }
    wait_vmem();  // no DMA may still target this workgroup's LDS when it is reused
  }
  __syncthreads();

  const float ltot = l + xor_lane(l, 32);
  if (t.splits == 1) {
    if (row < t.C) {
      const float inv = 1.0f / ltot;
      char* orow = reinterpret_cast<char*>(p.op) + ((int64_t)(t.row_base + row) * p.hq + t.head) * D * 2;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          uint2 w;
          w.x = pack_bf16(o[db][4 * jq] * inv, o[db][4 * jq + 1] * inv);
          w.y = pack_bf16(o[db][4 * jq + 2] * inv, o[db][4 * jq + 3] * inv);
          *reinterpret_cast<uint2*>(orow + (32 * db + 8 * jq + 4 * half) * 2) = w;
        }
    }
    return;
  }
  // split partial: unnormalised acc, m (base 2), l
  using Rc = PfRec<D, C::RPW>;
  const int w = wave_id();
  const Rsrc rs = dev_rsrc(reinterpret_cast<const char*>(p.p_part) + (int64_t)task * Rc::BYTES, Rc::BYTES);
  const uint32_t ro = Rc::acc_off(w) + rl * D * 4;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int jq = 0; jq < 4; ++jq)
      st_dev4(rs, ro + (32 * db + 8 * jq + 4 * half) * 4, o[db][4 * jq], o[db][4 * jq + 1], o[db][4 * jq + 2],
              o[db][4 * jq + 3]);
  if (half == 0) {
    st_dev1(rs, Rc::m_off(w) + rl * 4, m);
    st_dev1(rs, Rc::l_off(w) + rl * 4, ltot);
  }
  prefill_finish_split<Bf16, D, C::RPW>(p, t, task, lb);
}

// bf16 prefill tile of the four-workgroups-per-CU envelope (at most 128
// registers per lane, 40 KB of LDS per workgroup): 16 query rows of one
// head per wave on v_mfma_f32_16x16x32_bf16, the same 32-key blocks and
// LDS-DMA staging as the 32-row tile but through two stages, one block
// ahead.  Per block:
//   S^T[key, row] = K Q^T      two 16-key tiles x D/32 k-steps; A = K rows
//                              from LDS, B = Q^T in registers;
//   O^T[d, row] += V^T P^T     D/16 d tiles, the block's 32 keys as k; A =
//                              V^T from two transposing reads (keys 4q..4q+3
//                              and 16+4q..16+4q+3), B = P^T straight from the
//                              S^T accumulators (the key order is permuted
//                              the same way on both sides).
// Lane l holds row l & 15; the four lanes of a row (quads q = l >> 4) hold
// different keys and share the running maximum, raised lazily as in the
// 32-row tile.
template <int D>
struct PfBf16x4 {
  static constexpr int RPW = 16;                     // query rows per wave
  static constexpr int BN = PfBf16<D>::BN;           // keys per staged block
  static constexpr int ROWB = D * 2;
  static constexpr int OPB = BN * ROWB;              // bytes per operand per stage
  static constexpr int STAGE = 2 * OPB;              // K block then V block
  static constexpr int CH = D / 8;
  static_assert(2 * DecMfma4<D>::LDS_WAVE <= STAGE, "two decode waves share a stage buffer");
};

template <int D>
DEV void prefill_tile_bf16x4(const PodParams& p, int task, const LdsBufs& lb) {
  using C = PfBf16x4<D>;
  constexpr int KC = D / 32;   // QK k-steps
  constexpr int DT = D / 16;   // 16-wide d tiles of O^T
  const TaskGeom t = prefill_geom<C::RPW>(p, task);
  const int lane = lane_id();
  const int q4 = lane >> 4, rl = lane & 15;
  const int row = t.row0 + rl;
  const int64_t tok_bytes = (int64_t)p.hkv * D * 2;
  const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)t.g * D * 2;
  const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)t.g * D * 2;
  char* stg[2] = {lb.st[0], lb.st[2]};

  // Q^T operand: lane holds d = 32c + 8 q4 .. +8 of its row
  bf16x8_t qf[KC];
  {
    const char* qrow =
        reinterpret_cast<const char*>(p.qp) + (((int64_t)(t.row_base + row) * p.hq + t.head) * D + 8 * q4) * 2;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row < t.C) v = *reinterpret_cast<const uint4*>(qrow + c * 64);
      qf[c] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  f32x4_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.0f;

  const int nblk = t.k1 > t.k0 ? (t.k1 - t.k0 + C::BN - 1) / C::BN : 0;
  const int lim = t.P0 + row;  // last visible key of this lane's row

  int* pids = lb.pids;
  const int pg0 = t.k0 / kPageSize;
  const int pg1 = min((t.Lp + kPageSize - 1) / kPageSize, (t.k0 + nblk * C::BN + kPageSize - 1) / kPageSize);
  preload_page_ids(t.pt, p.num_pages, pg0, pg1 - pg0, pids);
  __syncthreads();

  if (nblk > 0) {
    const PfDma<D> dma = prefill_dma_offsets<D, true>(tok_bytes);
    auto kb_of = [&](int b) __attribute__((always_inline)) { return t.k0 + min(b, nblk - 1) * C::BN; };
    prefill_issue_block<D, true>(kpool, vpool, tok_bytes,
                                 __builtin_amdgcn_readfirstlane(pids[prefill_wave_page_index<D>(kb_of(0), t.Lp, pg0)]),
                                 t.Lp, kb_of(0), dma, stg[0]);
    int pid_next = pids[prefill_wave_page_index<D>(kb_of(1), t.Lp, pg0)];
    // Per-lane operand offsets inside a stage.  K: row rl of each 16-key tile
    // (the second tile 16 rows further: the swizzle depends on row & 15
    // only), chunk 4c + q4.  V: key rows 4 q4 + tk and 16 + 4 q4 + tk,
    // d = 16 dt + 4 tj .. +4.  Masked to 16 bits so that the stage base
    // folds into the reads' immediate offsets.
    uint32_t koff[KC], voff[DT];
    const int tk = rl >> 2, tj = rl & 3;
    const int vr0 = 4 * q4 + tk;
#pragma unroll
    for (int c = 0; c < KC; ++c) koff[c] = (uint32_t)(rl * C::ROWB + (((4 * c + q4) ^ ksw_rows<C::CH>(rl)) << 4)) & 0xffffu;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      voff[dt] = (uint32_t)(C::OPB + vr0 * C::ROWB + (((2 * dt + (tj >> 1)) ^ vsw_decode<C::CH>(vr0)) << 4) + ((tj & 1) << 3)) & 0xffffu;
    const float c2 = p.scale_log2;

    for (int b = 0; b < nblk; ++b) {
      // block b has landed (this wave's share) and, after the barrier, every
      // wave's share; every wave is also done with block b - 1, whose stage
      // the next DMA overwrites
      wait_vm_lgkm<0>();
      __builtin_amdgcn_s_barrier();
      const int page = __builtin_amdgcn_readfirstlane(pid_next);
      prefill_issue_block<D, true>(kpool, vpool, tok_bytes, page, t.Lp, kb_of(b + 1), dma, stg[(b + 1) & 1]);
      pid_next = pids[prefill_wave_page_index<D>(kb_of(b + 2), t.Lp, pg0)];
      const char* st = stg[b & 1];
      const int kb0 = t.k0 + b * C::BN;
      // S^T of the block's two 16-key tiles; one tile's K operands in
      // registers at a time (the envelope has 128 registers per lane)
      f32x4_t sc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sc[tt] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
        bf16x8_t ka[KC];
#pragma unroll
        for (int c = 0; c < KC; ++c) ka[c] = *reinterpret_cast<const bf16x8_t*>(st + koff[c] + tt * 16 * C::ROWB);
#pragma unroll
        for (int c = 0; c < KC; ++c) sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[c], qf[c], sc[tt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if ((kb0 + C::BN - 1) > (t.P0 + t.row0)) {  // diagonal block: causal mask
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 4; ++j) sc[tt][j] = kb0 + 16 * tt + 4 * q4 + j <= lim ? sc[tt][j] : kNegInf;
      }
      float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
      mx = fmaxf(mx, fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      mx *= c2;  // scale > 0: the max commutes with it
      if (__builtin_amdgcn_ballot_w64(mx > m + 8.0f) != 0) {
        const float mm = max_xor32(max_xor16(mx));
        const float mnew = fmaxf(m, mm);
        const float alpha = fast_exp2(m - safe_max(mnew));
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        m = mnew;
      }
      const float nmu = -safe_max(m);
      uint32_t pw[4];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
          pw[2 * tt + q2] = pack_bf16(fast_exp2(fmaf(sc[tt][2 * q2], c2, nmu)), fast_exp2(fmaf(sc[tt][2 * q2 + 1], c2, nmu)));
          // l sums the bf16 weights the PV product uses, so they normalise exactly
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[2 * tt + q2]), kOnes2, l, false);
        }
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      // PV in groups of two d tiles (their V^T operands read together)
      constexpr int DG = 2;
#pragma unroll
      for (int d0 = 0; d0 < DT; d0 += DG) {
        bf16x8_t va[DG];
#pragma unroll
        for (int e = 0; e < DG; ++e) {
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(st + voff[d0 + e]));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(st + voff[d0 + e] + 16 * C::ROWB));
          va[e] = __builtin_bit_cast(bf16x8_t, (short __attribute__((ext_vector_type(8)))){
              lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
#pragma unroll
        for (int e = 0; e < DG; ++e) o[d0 + e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[e], pf, o[d0 + e], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    wait_vmem();  // no DMA may still target this workgroup's LDS when it is reused
  }
  __syncthreads();

  const float ltot = sum_xor32(sum_xor16(l));
  if (t.splits == 1) {
    if (row < t.C) {
      const float inv = 1.0f / ltot;
      char* orow = reinterpret_cast<char*>(p.op) + (((int64_t)(t.row_base + row) * p.hq + t.head) * D + 4 * q4) * 2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        uint2 w;
        w.x = pack_bf16(o[dt][0] * inv, o[dt][1] * inv);
        w.y = pack_bf16(o[dt][2] * inv, o[dt][3] * inv);
        *reinterpret_cast<uint2*>(orow + 32 * dt) = w;
      }
    }
    return;
  }
  // split partial: unnormalised acc, m (base 2), l
  using Rc = PfRec<D, C::RPW>;
  const int w = wave_id();
  const Rsrc rs = dev_rsrc(reinterpret_cast<const char*>(p.p_part) + (int64_t)task * Rc::BYTES, Rc::BYTES);
  const uint32_t ro = Rc::acc_off(w) + rl * D * 4;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st_dev4(rs, ro + (16 * dt + 4 * q4) * 4, o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
  if (q4 == 0) {
    st_dev1(rs, Rc::m_off(w) + rl * 4, m);
    st_dev1(rs, Rc::l_off(w) + rl * 4, ltot);
  }
  prefill_finish_split<Bf16, D, C::RPW>(p, t, task, lb);
}

// fp32 prefill tile (exact fp32, VALU): lane = one query row, K/V blocks of 32
// keys in LDS read as broadcasts.
template <int D>
struct PfF32 {
  static constexpr int RPW = 64;
  static constexpr int BN = 32;
  static constexpr int STAGE = BN * D * 4;  // one operand block per stage buffer
};

template <int D>
DEV void prefill_tile_f32(const PodParams& p, int task, const LdsBufs& lb) {
  using C = PfF32<D>;
  const TaskGeom t = prefill_geom<C::RPW>(p, task);
  const int lane = lane_id();
  const int row = t.row0 + lane;
  float* ks = reinterpret_cast<float*>(lb.st[0]);
  float* vs = reinterpret_cast<float*>(lb.st[1]);

  float q[D], acc[D];
  {
    const float* qrow = reinterpret_cast<const float*>(p.qp) + ((int64_t)(t.row_base + row) * p.hq + t.head) * D;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      float4 v = make_float4(0, 0, 0, 0);
      if (row < t.C) v = *reinterpret_cast<const float4*>(qrow + e);
      q[e] = v.x;
      q[e + 1] = v.y;
      q[e + 2] = v.z;
      q[e + 3] = v.w;
    }
  }
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.0f;
  float m = kNegInf, l = 0.0f;
  const int lim = t.P0 + row;
  const int nblk = t.k1 > t.k0 ? (t.k1 - t.k0 + C::BN - 1) / C::BN : 0;
  const int64_t tok = (int64_t)p.hkv * D;
  const float* kpool = reinterpret_cast<const float*>(p.k_pool) + (int64_t)t.g * D;
  const float* vpool = reinterpret_cast<const float*>(p.v_pool) + (int64_t)t.g * D;
  constexpr int V4 = C::BN * D / 4;  // float4 chunks per operand block
  for (int b = 0; b < nblk; ++b) {
    const int kb0 = t.k0 + b * C::BN;
    __syncthreads();
    for (int idx = threadIdx.x; idx < V4; idx += 256) {
      const int kk = idx / (D / 4), c = idx % (D / 4);
      const int key = kb0 + kk;
      float4 kv = make_float4(0, 0, 0, 0), vv = kv;
      if (key < t.Lp) {
        const int64_t page = min((uint32_t)t.pt[key >> 4], p.num_pages - 1u);
        const int64_t off = (page * kPageSize + (key & 15)) * tok + 4 * c;
        kv = *reinterpret_cast<const float4*>(kpool + off);
        vv = *reinterpret_cast<const float4*>(vpool + off);
      }
      reinterpret_cast<float4*>(ks)[idx] = kv;
      reinterpret_cast<float4*>(vs)[idx] = vv;
    }
    __syncthreads();
    if (kb0 >= t.kw) continue;
    float s[C::BN];
    float mx = kNegInf;
#pragma unroll
    for (int kk = 0; kk < C::BN; ++kk) {
      float a = 0.0f;
#pragma unroll
      for (int e = 0; e < D; ++e) a = fmaf(q[e], ks[kk * D + e], a);
      a *= p.scale_log2;
      a = (kb0 + kk <= lim) ? a : kNegInf;
      s[kk] = a;
      mx = fmaxf(mx, a);
    }
    const float mnew = fmaxf(m, mx);
    const float mu = safe_max(mnew);
    const float alpha = fast_exp2(m - mu);
    float ps = 0.0f;
#pragma unroll
    for (int kk = 0; kk < C::BN; ++kk) {
      s[kk] = fast_exp2(s[kk] - mu);
      ps += s[kk];
    }
    l = l * alpha + ps;
    m = mnew;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      float a = acc[e] * alpha;
#pragma unroll
      for (int kk = 0; kk < C::BN; ++kk) a = fmaf(s[kk], vs[kk * D + e], a);
      acc[e] = a;
    }
  }
  if (t.splits == 1) {
    if (row < t.C) {
      const float inv = 1.0f / l;
      float* orow = reinterpret_cast<float*>(p.op) + ((int64_t)(t.row_base + row) * p.hq + t.head) * D;
#pragma unroll
      for (int e = 0; e < D; e += 4)
        *reinterpret_cast<float4*>(orow + e) = make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    }
    return;
  }
  using Rc = PfRec<D, C::RPW>;
  const int w = wave_id();
  const Rsrc rs = dev_rsrc(reinterpret_cast<const char*>(p.p_part) + (int64_t)task * Rc::BYTES, Rc::BYTES);
  const uint32_t ro = Rc::acc_off(w) + lane * D * 4;
#pragma unroll
  for (int e = 0; e < D; e += 4) st_dev4(rs, ro + e * 4, acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  st_dev1(rs, Rc::m_off(w) + lane * 4, m);
  st_dev1(rs, Rc::l_off(w) + lane * 4, l);
  prefill_finish_split<F32, D, C::RPW>(p, t, task, lb);
}

template <class E, int D>
struct PfSel;
template <int D>
struct PfSel<Bf16, D> {
  static constexpr int STAGE = PfBf16<D>::STAGE;
  // Where a prefill tile shares a SIMD with decode waves, it issues first
  // unless the plan says otherwise: its matrix and vector work is the longer
  // pole, while a decode wave mostly waits on memory (measured: ~1% faster
  // on the long-context batch; the opposite order made it ~13% slower).
  static DEV void run(const PodParams& p, int task, const LdsBufs& lb) {
    if (p.prefill_priority) __builtin_amdgcn_s_setprio(1);
    prefill_tile_bf16<D>(p, task, lb);
    __builtin_amdgcn_s_setprio(0);
  }
};
template <int D>
struct PfSel<F32, D> {
  static constexpr int STAGE = PfF32<D>::STAGE;
  static DEV void run(const PodParams& p, int task, const LdsBufs& lb) { prefill_tile_f32<D>(p, task, lb); }
};

// Stage buffer size: large enough for a prefill stage and a decode wave's V pages.
template <class E, int D>
constexpr int stage_bytes() {
  return PfSel<E, D>::STAGE > DecMfma<D>::LDS_WAVE ? PfSel<E, D>::STAGE : DecMfma<D>::LDS_WAVE;
}

#define POD_DECLARE_LDS(E, D)                                                          \
  __shared__ __attribute__((aligned(16))) char lds_st0[stage_bytes<E, D>()];             \
  __shared__ __attribute__((aligned(16))) char lds_st1[stage_bytes<E, D>()];             \
  __shared__ __attribute__((aligned(16))) char lds_st2[stage_bytes<E, D>()];             \
  __shared__ __attribute__((aligned(16))) char lds_st3[stage_bytes<E, D>()];             \
  __shared__ int lds_pids[kMaxSplitKeys / kPageSize];                                    \
  __shared__ int lds_flag;                                                               \
  const LdsBufs lb{{lds_st0, lds_st1, lds_st2, lds_st3}, lds_pids, &lds_flag}

// LDS of the four-workgroups-per-CU envelope: two prefill stages (each
// also holding two decode waves' page buffers) and the split's page ids.
#define POD_DECLARE_LDS4(D)                                                                          \
  __shared__ __attribute__((aligned(16))) char lds4_s0[PfBf16x4<D>::STAGE];                          \
  __shared__ __attribute__((aligned(16))) char lds4_s1[PfBf16x4<D>::STAGE];                          \
  __shared__ int lds_pids[kMaxSplitKeys / kPageSize];                                                \
  __shared__ int lds_flag;                                                                           \
  const LdsBufs lb{{lds4_s0, lds4_s0 + PfBf16x4<D>::STAGE / 2, lds4_s1, lds4_s1 + PfBf16x4<D>::STAGE / 2}, \
                   lds_pids, &lds_flag}

// ------------------------------------------------------------------ kernels
// Pages in flight per decode wave: the fused kernel keeps 2 WGs per CU, so its
// decode waves prefetch deeper; the decode-only kernel runs more waves instead.
template <class E, int G>
constexpr int fused_pf() { return E::bytes == 2 ? 1 : (G >= 8 ? 1 : 2); }  // bf16: pairs of pages
template <class E>
constexpr int decode_pf() { return 1; }
template <class E, int G>
constexpr int decode_min_blocks() { return E::bytes == 2 ? 2 : (G >= 4 ? 2 : 4); }

template <class E, int D, int G>
__global__ __launch_bounds__(256, 2) void pod_prefill_kernel(PodParams p) {
  POD_DECLARE_LDS(E, D);
  PfSel<E, D>::run(p, blockIdx.x, lb);
}

template <class E, int D, int G>
__global__ __launch_bounds__(256, (decode_min_blocks<E, G>())) void pod_decode_kernel(PodParams p) {
  constexpr int W = E::bytes == 2 ? DecMfma<D>::LDS_WAVE : kMergeLdsBytes;  // per wave
  __shared__ __attribute__((aligned(16))) char dbuf0[W];
  __shared__ __attribute__((aligned(16))) char dbuf1[W];
  __shared__ __attribute__((aligned(16))) char dbuf2[W];
  __shared__ __attribute__((aligned(16))) char dbuf3[W];
  const LdsBufs lb{{dbuf0, dbuf1, dbuf2, dbuf3}, nullptr, nullptr};
  decode_wg<E, D, G, decode_pf<E>(), kRemBuckets>(p, blockIdx.x, lb);
}

// Per-XCD task queues: queue x of `heads` holds tasks x, x+8, x+16, ... of
// n.  A claim first bumps the claimer's own queue (one atomic; a head past
// the end is harmless, it is only compared), so claims spread over eight
// words instead of contending on one; once that queue is empty the other
// heads are read together and a non-empty queue is tried.  Prefill tasks are
// ordered kv head fastest, so with 8 kv heads each XCD streams one kv head's
// keys through its own L2.  n if every queue is empty; `done` then records
// it so later workgroups need not look again.
DEV uint32_t ctrl_load(const uint32_t* w) {
  return __hip_atomic_load(const_cast<uint32_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV uint32_t xcd_queue_len(uint32_t n, uint32_t x) {
  return n > x ? (n - x + kXcdQueues - 1) / kXcdQueues : 0u;
}
DEV uint32_t claim_xcd(uint32_t* heads, uint32_t* done, uint32_t n, uint32_t xcc) {
  uint32_t i = atomicAdd(heads + xcc, 1u);
  if (i < xcd_queue_len(n, xcc)) return xcc + kXcdQueues * i;
  uint32_t h[kXcdQueues];
#pragma unroll
  for (int x = 0; x < kXcdQueues; ++x) h[x] = ctrl_load(heads + x);
  for (int k = 1; k < kXcdQueues; ++k) {
    const uint32_t x = (xcc + k) % kXcdQueues;
    if (h[x] >= xcd_queue_len(n, x)) continue;
    i = atomicAdd(heads + x, 1u);
    if (i < xcd_queue_len(n, x)) return x + kXcdQueues * i;
  }
  __hip_atomic_store(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return n;
}

DEV bool claim_prefill(const PodParams& p, uint32_t xcc, int& task) {
  const uint32_t t = claim_xcd(p.ctrl + kCtrlPrefillHeads, p.ctrl + kCtrlPrefillDone, (uint32_t)p.p_tasks, xcc);
  task = (int)t;
  return t < (uint32_t)p.p_tasks;
}

DEV bool claim_decode(const PodParams& p, uint32_t xcc, int& task) {
  const uint32_t t = claim_xcd(p.ctrl + kCtrlDecodeHeads, p.ctrl + kCtrlDecodeDone, (uint32_t)p.d_wg_tasks, xcc);
  task = (int)t;
  return t < (uint32_t)p.d_wg_tasks;
}

// Role choice and task claim of one workgroup (thread 0) under the policies
// below.  Sets `task` past its role's count when both queues are empty.
DEV void pick_and_claim(const PodParams& p, int& role, int& task, bool& counted, uint32_t& key) {
  key = cu_key();
  const uint32_t xcc = (key >> 8) & 7u;
  uint32_t* word = p.tickets + key;
  counted = p.policy == kPolicyCuBalanced;
  if (p.policy == kPolicyCuBalanced) {
    const uint32_t frac = ((key * 2654435761u) >> 24) & 255u;
    const uint32_t target = ((uint32_t)p.cu_prefill_x256 >> 8) + (frac < ((uint32_t)p.cu_prefill_x256 & 255u) ? 1u : 0u);
    uint32_t old = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t pdone = ctrl_load(p.ctrl + kCtrlPrefillDone), ddone = ctrl_load(p.ctrl + kCtrlDecodeDone);
    if (pdone | ddone) {
      // one queue is empty: take the other, uncounted (the mix no longer matters)
      role = pdone ? 1 : 0;
      counted = false;
    } else {
      while (true) {
        role = (old & 0xffffu) < target ? 0 : 1;
        const uint32_t nw = old + (role == 0 ? 1u : 0x10000u);
        if (__hip_atomic_compare_exchange_strong(word, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
          break;
      }
    }
  } else if (p.policy == kPolicyStatic) {
    // (persistent grid only) prefill until its queue is empty, then decode
    role = ctrl_load(p.ctrl + kCtrlPrefillDone) ? 1 : 0;
  } else {
    const uint32_t t = atomicAdd(word, 1u) % (uint32_t)p.share_den;
    const uint32_t num = (uint32_t)p.share_num, den = (uint32_t)p.share_den;
    role = ((t + 1) * num + den - 1) / den > (t * num + den - 1) / den ? 0 : 1;
  }
  const int want = role;
  bool ok = role == 0 ? claim_prefill(p, xcc, task) : claim_decode(p, xcc, task);
  if (!ok) {
    role ^= 1;
    ok = role == 0 ? claim_prefill(p, xcc, task) : claim_decode(p, xcc, task);
  }
  if (!ok && counted) {  // nothing left: undo the count
    atomicSub(word, want == 0 ? 1u : 0x10000u);
    counted = false;
  } else if (counted && role != want) {  // recount under the role actually taken
    atomicAdd(word, role == 0 ? 1u - 0x10000u : 0x10000u - 1u);
  }
}

// Thread 0 of a workgroup that is done claiming: count it out; the last of
// the launch's workgroups clears the control words for the next launch.
// Every claim is a returning device-scope atomic and the flag stores are
// complete (vmcnt 0) before the count, so the clear lands after all of them
// without cache maintenance (an acquire-release count here, which writes
// back and invalidates the L2, made the fused launch 3-7% slower).
// Returns true for that last workgroup.
DEV bool leave_claims(const PodParams& p) {
  wait_vmem();
  const uint32_t n = __hip_atomic_fetch_add(p.ctrl + kCtrlExit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (n != (uint32_t)p.grid - 1u) return false;
  for (int q = 0; q < kCtrlUsed; ++q) __hip_atomic_store(p.ctrl + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// Under the ticket policies the per-CU words count arrivals and are never
// counted down by their workgroups; the last workgroup out of a launch (all
// claims are done by then) clears them with all its threads, so the next
// launch starts its ticket sequences at zero like the first one did.
DEV void clear_tickets(const PodParams& p) {
  for (int i = threadIdx.x; i < kTicketSlots; i += blockDim.x)
    __hip_atomic_store(p.tickets + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
DEV bool ticket_policy(const PodParams& p) {
  return p.policy == kPolicyProportional || p.policy == kPolicyHalf;
}

// Fused hybrid kernel.  A regular grid of prefill tasks + decode workgroup
// tasks is launched; each workgroup picks its role after dispatch from the
// compute unit it landed on (paper §4.1) and then claims a task of that role,
// or of the other role once the first is exhausted.  Since the grid equals
// the task count every claim succeeds, every task runs exactly once, and no
// workgroup ever waits for another.
//   CU-balanced (default): the CU's word counts running prefill (low half)
//     and decode (high half) workgroups; a workgroup takes prefill while
//     fewer than the CU's prefill target run there, decode otherwise, and
//     uncounts itself when done.  The targets are floor(x) or floor(x)+1
//     per CU (by a hash of the CU id) so that they average x =
//     cu_prefill_x256 / 256 over the chip.
//   proportional / half: the CU's ticket counter; ticket t mod share_den
//     runs prefill for share_num of every share_den arrivals, prefill first
//     (paper §5.4.2).
//   static: workgroup id decides, without looking at the CU (paper §3.3).
// A CU-balanced launch resident in one round (fixed_order) also hands out
// roles by workgroup id -- one role's tasks first, then the other's -- with
// no atomics in front of the work.
// Role trace: one 32-byte record per task of a fused launch (the realised
// mix of virtual workgroups, which the Silicon & Systems digest asks the
// runtime to report): the key of the CU it ran on, its role and task, and
// its start and end on the chip-wide 100 MHz real-time counter.  Written by
// thread 0 with plain vector stores once the task is done.
DEV void trace_task(const PodParams& p, int role, int task, uint32_t key, uint64_t t0) {
  const uint64_t t1 = __builtin_amdgcn_s_memrealtime();
  const int slot = role == 0 ? task : p.p_tasks + task;
  uint4* r = reinterpret_cast<uint4*>(p.trace + (int64_t)slot * 32);
  r[0] = make_uint4(key, (uint32_t)role, (uint32_t)task, 0u);
  r[1] = make_uint4((uint32_t)t0, (uint32_t)(t0 >> 32), (uint32_t)t1, (uint32_t)(t1 >> 32));
}

template <class RunP, class RunD>
DEV void fused_body(const PodParams& p, RunP&& run_prefill, RunD&& run_decode) {
  __shared__ int role_task[4];
  __shared__ uint32_t cu_word;
  if (threadIdx.x == 0) {
    int role, task = 0;
    bool counted = false, last = false;
    uint32_t key = 0;
    if (p.policy == kPolicyStatic) {
      role = (int)blockIdx.x < p.p_tasks ? 0 : 1;
      task = role == 0 ? (int)blockIdx.x : (int)blockIdx.x - p.p_tasks;
    } else if (p.fixed_order) {
      const int first = p.fixed_order == 2 ? 1 : 0;
      const int n_first = first == 1 ? p.d_wg_tasks : p.p_tasks;
      role = (int)blockIdx.x < n_first ? first : 1 - first;
      task = role == first ? (int)blockIdx.x : (int)blockIdx.x - n_first;
    } else {
      pick_and_claim(p, role, task, counted, key);
      last = leave_claims(p);  // one claim per workgroup
    }
    if (p.trace && !key) key = cu_key();
    cu_word = key;
    role_task[0] = role;
    role_task[1] = task;
    role_task[2] = counted;
    role_task[3] = last;
  }
  __syncthreads();
  const uint64_t t0 = p.trace ? __builtin_amdgcn_s_memrealtime() : 0;
  const int role = role_task[0], task = role_task[1];
  if (role_task[3] && ticket_policy(p)) clear_tickets(p);
  bool ran = false;
  if (role == 0) {
    if (task < p.p_tasks) {
      run_prefill(task);
      ran = true;
    }
  } else {
    if (task < p.d_wg_tasks) {
      run_decode(task);
      ran = true;
    }
  }
  if (role_task[2] || p.trace) {
    __syncthreads();
    if (threadIdx.x == 0) {
      if (role_task[2]) atomicSub(p.tickets + cu_word, role == 0 ? 1u : 0x10000u);
      if (p.trace && ran) trace_task(p, role, task, cu_word, t0);
    }
  }
}

// RB: remainder phases of the decode unit numbering (1: request order;
// kRemBuckets: longest first in length classes, for decode-first launches of
// several rounds, as in decode-only launches).
template <class E, int D, int G, int RB = 1>
__global__ __launch_bounds__(256, 2) void pod_hybrid_kernel(PodParams p) {
  POD_DECLARE_LDS(E, D);
  fused_body(
      p, [&](int task) { PfSel<E, D>::run(p, task, lb); },
      [&](int task) { decode_wg<E, D, G, fused_pf<E, G>(), RB>(p, task, lb); });
}

// The three launches of the four-workgroups-per-CU envelope (bf16 only).
template <int D, int G>
__global__ __launch_bounds__(256, 4) void pod_hybrid4_kernel(PodParams p) {
  POD_DECLARE_LDS4(D);
  fused_body(
      p,
      [&](int task) {
        if (p.prefill_priority) __builtin_amdgcn_s_setprio(1);
        prefill_tile_bf16x4<D>(p, task, lb);
        __builtin_amdgcn_s_setprio(0);
      },
      [&](int task) { decode_wg4<D, G>(p, task, lb); });
}

template <int D, int G>
__global__ __launch_bounds__(256, 4) void pod_prefill4_kernel(PodParams p) {
  POD_DECLARE_LDS4(D);
  prefill_tile_bf16x4<D>(p, blockIdx.x, lb);
}

template <int D, int G>
__global__ __launch_bounds__(256, 4) void pod_decode4_kernel(PodParams p) {
  constexpr int W = DecMfma4<D>::LDS_WAVE;
  __shared__ __attribute__((aligned(16))) char dbuf0[W];
  __shared__ __attribute__((aligned(16))) char dbuf1[W];
  __shared__ __attribute__((aligned(16))) char dbuf2[W];
  __shared__ __attribute__((aligned(16))) char dbuf3[W];
  __shared__ int dpids[kWavesPerWG * kSplitIdRegs * 64];
  const LdsBufs lb{{dbuf0, dbuf1, dbuf2, dbuf3}, dpids, nullptr};
  decode_wg4<D, G, kRemBuckets>(p, blockIdx.x, lb);
}

// Persistent variant of the fused kernel: a grid of (CUs x resident
// workgroups) that loops — pick a role by the policy, claim a task of it,
// run it, uncount — until both queues are empty (paper §4.3 mentions such a
// variant performing on par).  Same tasks, same merges, same results.
template <class E, int D, int G>
__global__ __launch_bounds__(256, 2) void pod_persistent_kernel(PodParams p) {
  POD_DECLARE_LDS(E, D);
  __shared__ int role_task[4];
  __shared__ uint32_t cu_word;
  while (true) {
    if (threadIdx.x == 0) {
      int role, task = 0;
      bool counted, last = false;
      uint32_t key;
      pick_and_claim(p, role, task, counted, key);
      if (task >= (role == 0 ? p.p_tasks : p.d_wg_tasks)) last = leave_claims(p);  // both queues empty
      cu_word = key;
      role_task[0] = role;
      role_task[1] = task;
      role_task[2] = counted;
      role_task[3] = last;
    }
    __syncthreads();
    const uint64_t t0 = p.trace ? __builtin_amdgcn_s_memrealtime() : 0;
    const int role = role_task[0], task = role_task[1];
    if (role_task[3] && ticket_policy(p)) clear_tickets(p);
    if (role == 0) {
      if (task >= p.p_tasks) break;  // both queues empty (uniform: read from LDS)
      PfSel<E, D>::run(p, task, lb);
    } else {
      if (task >= p.d_wg_tasks) break;
      decode_wg<E, D, G, fused_pf<E, G>()>(p, task, lb);
    }
    __syncthreads();  // the task's LDS and role_task are free again
    if (threadIdx.x == 0 && role_task[2]) atomicSub(p.tickets + cu_word, role == 0 ? 1u : 0x10000u);
    if (threadIdx.x == 0 && p.trace) trace_task(p, role, task, cu_word ? cu_word : cu_key(), t0);
  }
}

// ------------------------------------------------------------------- launch
template <class E, int D, int G>
static int launch_t(int which, const PodParams& p, const Plan& pl, hipStream_t s) {
  const dim3 block(256);
  // the decode units were numbered for the kernel family that runs them:
  // length classes in decode-only launches and in decode-first fused
  // launches of several rounds in the two-workgroup grid, request order in
  // other fused ones (the kernels fix the class count at compile time)
  if (pl.has_d) {
    const bool classes = pl.rem_buckets == kRemBuckets;
    if (!classes && pl.rem_buckets != 1) return (int)hipErrorInvalidValue;
    if (which == kKernelDecode && !classes) return (int)hipErrorInvalidValue;
    if (which == kKernelHybrid && classes && (pl.wg_per_cu != 2 || pl.persistent)) return (int)hipErrorInvalidValue;
  }
  if (pl.wg_per_cu == 4) {
    if constexpr (E::bytes == 2) {
      switch (which) {
        case kKernelHybrid:
          hipLaunchKernelGGL((pod_hybrid4_kernel<D, G>), dim3(pl.grid), block, 0, s, p);
          break;
        case kKernelPrefill:
          hipLaunchKernelGGL((pod_prefill4_kernel<D, G>), dim3(pl.p_tasks), block, 0, s, p);
          break;
        default:
          hipLaunchKernelGGL((pod_decode4_kernel<D, G>), dim3(pl.d_wg_tasks), block, 0, s, p);
          break;
      }
      return (int)hipGetLastError();
    }
    return (int)hipErrorInvalidValue;
  }
  switch (which) {
    case kKernelHybrid:
      if (pl.persistent)
        hipLaunchKernelGGL((pod_persistent_kernel<E, D, G>), dim3(pl.grid), block, 0, s, p);
      else if (pl.has_d && pl.rem_buckets == kRemBuckets)
        hipLaunchKernelGGL((pod_hybrid_kernel<E, D, G, kRemBuckets>), dim3(pl.grid), block, 0, s, p);
      else
        hipLaunchKernelGGL((pod_hybrid_kernel<E, D, G>), dim3(pl.grid), block, 0, s, p);
      break;
    case kKernelPrefill:
      hipLaunchKernelGGL((pod_prefill_kernel<E, D, G>), dim3(pl.p_tasks), block, 0, s, p);
      break;
    default:
      hipLaunchKernelGGL((pod_decode_kernel<E, D, G>), dim3(pl.d_wg_tasks), block, 0, s, p);
      break;
  }
  return (int)hipGetLastError();
}

#define POD_KERNEL_LIST(X)  \
  X(kBf16, Bf16, 128, 1)    \
  X(kBf16, Bf16, 128, 2)    \
  X(kBf16, Bf16, 128, 4)    \
  X(kBf16, Bf16, 128, 8)    \
  X(kBf16, Bf16, 64, 1)     \
  X(kBf16, Bf16, 64, 2)     \
  X(kBf16, Bf16, 64, 4)     \
  X(kBf16, Bf16, 64, 8)     \
  X(kF32, F32, 64, 1)       \
  X(kF32, F32, 64, 2)       \
  X(kF32, F32, 64, 4)       \
  X(kF32, F32, 64, 8)

int launch(int which, int dtype, int d, int G, const PodParams& p, const Plan& pl, hipStream_t s) {
#define POD_DISPATCH(DT, E, DD, GG) \
  if (dtype == DT && d == DD && G == GG) return launch_t<E, DD, GG>(which, p, pl, s);
  POD_KERNEL_LIST(POD_DISPATCH)
#undef POD_DISPATCH
  return (int)hipErrorInvalidValue;
}

// ------------------------------------------------- allocation-free scratch
// Workspace of pod_attn_hybrid_noalloc: a fixed array in the code object's
// device memory, one copy per GPU the library runs on, held until the
// process ends.  Calls on one GPU share it (and race if they overlap).
constexpr size_t kScratchBytes = POD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

size_t scratch_bytes() { return kScratchBytes; }

// The array's device address on `device`, looked up once per device with
// that device current (the host-side name of the array is not a device
// address and must never reach a kernel or a copy).
int scratch_address(int device, void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices || !out) return (int)hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != device) e = hipSetDevice(device);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != device) (void)hipSetDevice(cur);
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return 0;
}

__global__ __launch_bounds__(256) void pod_zero_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * 256u + threadIdx.x; i < n; i += gridDim.x * 256u) p[i] = 0u;
}

int launch_zero(void* p, size_t bytes, hipStream_t s) {
  const uint32_t n = (uint32_t)(bytes / 4);
  if (n == 0) return 0;
  const uint32_t blocks = (n + 255) / 256 < 1024u ? (n + 255) / 256 : 1024u;
  hipLaunchKernelGGL(pod_zero_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
  return (int)hipGetLastError();
}

// ------------------------------------------------ measured-peak kernels
// Two plain kernels that measure what the chip sustains, for a roofline
// fraction against measured rather than published peaks.
//
// HBM read: each wave streams its own contiguous slice of `wave_bytes`
// with nontemporal 16-byte buffer loads, two register buffers of 16 loads
// (16 KB) in flight, and folds what it reads with XOR.  Loads past the
// slice (the last buffer when the slice holds an odd count) return zeros
// and touch no memory.
constexpr int kPeakLoads = 16;

__global__ __launch_bounds__(256, 2) void pod_peak_read_kernel(const char* buf, uint32_t wave_bytes, uint32_t* sink) {
  const int w = threadIdx.x >> 6, lane = lane_id();
  const char* base = buf + ((uint64_t)blockIdx.x * kWavesPerWG + w) * wave_bytes;
  const Rsrc r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)wave_bytes, 0x00020000);
  const uint32_t nbuf = wave_bytes / (kPeakLoads * 1024u);
  u32x4_t b0[kPeakLoads], b1[kPeakLoads], acc = {0u, 0u, 0u, 0u};
  auto issue = [&](u32x4_t (&b)[kPeakLoads], uint32_t i) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPeakLoads; ++u)
      b[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(i * kPeakLoads * 1024u + u * 1024u + lane * 16u), 0,
                                                   kNonTemporal);
  };
  auto fold = [&](const u32x4_t (&b)[kPeakLoads]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPeakLoads; ++u) acc ^= b[u];
  };
  issue(b0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue(b1, 1);
  __builtin_amdgcn_sched_barrier(0);
  for (uint32_t i = 0; i < nbuf; i += 2) {
    fold(b0);
    issue(b0, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    fold(b1);
    issue(b1, i + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  // the store keeps the loads; it runs only if the XOR hits this constant
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) sink[0] = 1u;
}

// MFMA loop: four independent v_mfma_f32_32x32x16_bf16 chains per wave on
// register operands (no memory traffic), 16 MFMAs per iteration.
__global__ __launch_bounds__(256, 2) void pod_peak_mfma_kernel(int iters, uint32_t* sink) {
  const uint32_t lane = (uint32_t)lane_id();
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f003f80u ^ lane, 0x3e803f00u, 0x3f803c00u));
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, make_uint4(0x3c003f80u, 0x3f803f00u, 0x3f80u ^ (lane << 16), 0x3e803f80u));
  f32x16_t c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[k][j] = 0.0f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      c[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c[1], 0, 0, 0);
      c[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c[2], 0, 0, 0);
      c[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c[3], 0, 0, 0);
    }
  }
  float sum = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int j = 0; j < 16; ++j) sum += c[k][j];
  if (__float_as_uint(sum) == 0x9e3779b9u) sink[0] = 1u;
}

int launch_peak_read(const void* buf, size_t bytes, int workgroups, uint32_t* sink, hipStream_t s) {
  const uint64_t wave_bytes = bytes / ((uint64_t)workgroups * kWavesPerWG);
  hipLaunchKernelGGL(pod_peak_read_kernel, dim3(workgroups), dim3(256), 0, s, static_cast<const char*>(buf),
                     (uint32_t)wave_bytes, sink);
  return (int)hipGetLastError();
}

int launch_peak_mfma(int workgroups, int iters, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(pod_peak_mfma_kernel, dim3(workgroups), dim3(256), 0, s, iters, sink);
  return (int)hipGetLastError();
}

int have_kernel(int dtype, int d, int G) {
#define POD_HAVE(DT, E, DD, GG) \
  if (dtype == DT && d == DD && G == GG) return 1;
  POD_KERNEL_LIST(POD_HAVE)
#undef POD_HAVE
  return 0;
}

}  // namespace pod
