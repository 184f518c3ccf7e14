// attn_sink.hip -- gfx950 (MI355X) kernels and C ABI for grouped-query
// attention with per-head attention sinks.
//
// The operation (page "GPT-OSS on Day 0", perplexity.ai, sections
// "Attention: GQA with Attention Sinks" and "Kernels for GPT-OSS / Sink
// Attention"): each query head h owns a sink logit s_h that joins the softmax
// denominator and has no value row; query head h reads key/value head
// h / G.  The softmax runs online: a running max m that starts at the head's
// sink (not at -inf) and a running sum d that starts at e^(s - m) = 1, so the
// sink is accumulated exactly once.  The work is spread over heads and over
// blocks of the key length; when the key range is split, only the first
// block starts from the sink, and a merge combines the blocks' (m, d, o).
//
// Kernels (all hand-written for CDNA4, 64-lane wavefronts):
//   decode_kernel   paged decode, one query token per sequence.  One
//                   workgroup owns (sequence, kv head, key chunk); the G query
//                   heads of the group sit in the 16 columns of one MFMA tile,
//                   so every K and V page is loaded from HBM once for all of
//                   them.  Pages are read with non-temporal vector loads: V
//                   (stored dim-major, so that the P.V contraction over
//                   tokens reads contiguous memory) straight into MFMA
//                   operands, K as whole 128-byte rows re-dealt into the
//                   operand layout through 2 KB of LDS per wave.  The waves
//                   of a workgroup take interleaved pages of its chunk and
//                   merge their states in LDS; unsplit decode runs 16 waves
//                   per workgroup, so a sequence's whole key range is split
//                   and merged inside one launch without partial states.
//   merge_kernel    split-KV merge of (m, d, o) partial states.
//   prefill_kernel  ragged (causal) prefill.  One workgroup owns a tile of
//                   query tokens x all G heads of one kv head (4 waves x 64
//                   rows), so a K/V tile staged in LDS serves every head of
//                   the group.  S^T = K Q^T and O^T = V^T P^T run on 32x32
//                   MFMAs; the transposed products make the score tile's
//                   register layout directly usable as the P operand of the
//                   next product, and keep each query row's softmax state in
//                   the lane that owns that row.
//
// Internally logits are kept in log2 units (x * sm_scale * log2 e) so the
// exponentials are single v_exp_f32 instructions; the sink is converted by
// log2 e only (it is not multiplied by sm_scale).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>


#include "attn_sink.h"

// Device memory of attn_sink_decode_paged_static (see scratch_for below):
// the split partial states of one call, at most kScratchBytes.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kHeadDim = 64;
constexpr int kPage = 16;
// Prefill forms P against a lazily kept reference and moves the reference
// only when a lane's share of a tile's row sum exceeds this bound: P then
// stays below 2^64, so O and d (sums of P times values, up to 2^17 keys)
// stay far below the fp32 and bf16 range (2^128).
constexpr float kLaneSumMax = 0x1p64f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = ATTN_SINK_F32, DT_BF16 = ATTN_SINK_BF16 };

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor_max(float v, int mask) {
  return fmaxf(v, __shfl_xor(v, mask, 64));
}

__device__ __forceinline__ float xor_sum(float v, int mask) {
  return v + __shfl_xor(v, mask, 64);
}

// fp32 -> bf16 bits, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ unsigned short to_bf16(float x) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(x));
}

// Two fp32 -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned int, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}


// True on every lane if the predicate holds on any lane of the wave.
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xffff0000u); }

template <typename V>
__device__ __forceinline__ V ld_global(const void* p) {
  return *reinterpret_cast<const V*>(p);
}

// Load marked non-temporal: data read once (the paged decode's K and V) is
// streamed past the caches, which reads random 2 KB pages ~10% faster.
template <typename V>
__device__ __forceinline__ V ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero and stores past the end are dropped, which is how ragged sequence
// tails are handled without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Same with a wave-uniform part of the offset (held in an SGPR).
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                            uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Index of the sequence with the r-th largest length among n <= 64 (ties by
// index), one length per lane (lanes >= n hold -1): each lane counts the
// lengths that beat its own, one compare per lane and step.  r < n.
__device__ __forceinline__ int nth_longest(int len, int n, int r) {
  const int lane = threadIdx.x & 63;
  int rank = 0;
  for (int j = 0; j < n; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    rank += (lj > len) || (lj == len && j < lane);
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < n && rank == r);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
}

// Buffer resource words over [base, base + bytes) (the same descriptor as
// make_rsrc), for the loads issued from inline assembly below.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes
// [lds + 16 i, +16) (lds wave-uniform); offsets past the buffer read zero.
// Issued from inline assembly so that the compiler's wait insertion, which
// would wait for every such load before any LDS read, does not see it: the
// caller waits for these loads itself (vmcnt; loads complete in order).  The
// LDS address goes in M0, which is saved and restored around the load, with
// the one wait state gfx9 needs between an SALU write of M0 and its read.
__device__ __forceinline__ void load_to_lds16(u32x4 rsrc, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}

// Workgroup barrier ordering LDS only (global loads in flight stay in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// ============================================================ decode kernel
//
// Work item = (key chunk c, kv head, sequence b); WAVES waves share it by
// taking every WAVES-th page of the chunk, then merge their states in LDS.
// Per wave and page (16 tokens) the tile maths is
//   S^T[16 tok x 16 heads] = K[16 tok x 64] . Q^T[64 x 16 heads]
//   O^T[64 x 16 heads]    += V^T[64 x 16 tok] . P^T[16 tok x 16 heads]
// Register layout of a 16x16 MFMA result: lane l holds column l%16 (the
// head) and rows 4*(l/16) + r, r = 0..3 (tokens for S^T, dims for O^T), so
// each lane's softmax state belongs to exactly one head.

template <int DT>
struct DecodeFrag;

template <>
struct DecodeFrag<DT_BF16> {
  u32x4 k[2];  // as loaded: K[token 8s + l/8][8(l%8) .. +7], s = 0, 1
  u32x2 v[4];  // Vt[16j + l%16][4g .. 4g+3], j = 0..3
};

template <>
struct DecodeFrag<DT_F32> {
  u32x4 k[4];  // K[token l%16][16g .. 16g+15]
  u32x4 v[4];  // Vt[16j + l%16][4g .. 4g+3]
};

// Four bf16 decode waves per SIMD (at most 128 VGPRs), 16 per CU: two 8-wave
// split-decode workgroups or one 16-wave unsplit one keep that many pages in
// flight.
#ifndef ATTN_SINK_DECODE_MIN_WAVES
#define ATTN_SINK_DECODE_MIN_WAVES 4
#endif
template <int DT, int WAVES, int UNROLL>
__global__ __launch_bounds__(64 * WAVES, (DT == DT_BF16 ? ATTN_SINK_DECODE_MIN_WAVES : 1)) void decode_kernel(
    const char* __restrict__ q, const char* __restrict__ kc, const char* __restrict__ vc,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ kv_lens,
    const float* __restrict__ sinks, int max_pages, int num_pages, int hkv, int group,
    float qk_scale_log2, int splits, float* __restrict__ part_m, float* __restrict__ part_d,
    float* __restrict__ part_o, char* __restrict__ out) {
  constexpr int ES = DT == DT_BF16 ? 2 : 4;  // element size
  constexpr size_t kPageElems = (size_t)kPage * kHeadDim;
  const int c = blockIdx.x, kvh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  // Longest sequences first: workgroups are dispatched in blockIdx order, so
  // for up to 64 sequences blockIdx.z is read as a rank and mapped to the
  // sequence with the rank-th largest kv_len (ties by index).  The ranking
  // leaves every length in a register, so the sequence's own length costs no
  // second dependent load.
  int b = blockIdx.z, L;
  const int batch = gridDim.z;
  if (batch <= 64) {
    const int li = lane < batch ? clampi(kv_lens[lane], 0, max_pages * kPage) : -1;
    b = nth_longest(li, batch, (int)blockIdx.z);
    L = __builtin_amdgcn_readlane(li, b);
  } else {
    L = clampi(kv_lens[b], 0, max_pages * kPage);
  }
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int hq = hkv * group;
  const bool head_ok = n < group;
  const int h = kvh * group + (head_ok ? n : 0);

  const int np = (L + kPage - 1) / kPage;
  const int ppc = (np + splits - 1) / splits;
  const int p_begin = min(c * ppc, np);
  const int p_end = min(p_begin + ppc, np);

  // Q^T operand (B of S^T = K Q^T): this lane's head n, its k-slice of dims.
  const char* qrow = q + ((size_t)b * hq + h) * kHeadDim * ES;
  u32x4 qf[DT == DT_BF16 ? 2 : 4];
  if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
      qf[s] = head_ok ? ld_global<u32x4>(qrow + (32 * s + 8 * g) * ES) : u32x4{0, 0, 0, 0};
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[s] = head_ok ? ld_global<u32x4>(qrow + (16 * g + 4 * s) * ES) : u32x4{0, 0, 0, 0};
  }

  // Running state.  Chunk 0's first wave starts from the sink: m = s (log2
  // units), d = e^(s - m) = 1 (0 when s = -inf), counted in lane group 0 only
  // because d is summed over the four lane groups at the end.
  const float sink = head_ok ? sinks[h] : kNegInf;
  const bool carries_sink = (c == 0) && (w == 0);
  float m_run = carries_sink ? sink * kLog2e : kNegInf;
  float d_run = (carries_sink && g == 0 && sink != kNegInf) ? 1.0f : 0.0f;
  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* pt = page_table + (size_t)b * max_pages;
  const size_t head_page_stride = kPageElems * ES;  // bytes per (page, kv head)

  // bf16 K arrives as whole 128-byte token rows (load s, lane i: token
  // 8s + i/8, 16-byte chunk i%8) and is re-dealt into the MFMA operand
  // layout through a 2 KB LDS block per wave.  Chunk c of token t sits in
  // slot 8t + (c ^ ((t >> 1) & 7)), so the 16 lanes of each operand read
  // (tokens 0..15, one chunk) hit 16 different bank groups.
  __shared__ u32x4 k_lds[DT == DT_BF16 ? WAVES : 1][128];
  auto k_slot = [](int t, int ch) { return 8 * t + (ch ^ ((t >> 1) & 7)); };
  auto load_page = [&](int phys, DecodeFrag<DT>& f) {
    const char* kp = kc + ((size_t)phys * hkv + kvh) * head_page_stride;
    const char* vp = vc + ((size_t)phys * hkv + kvh) * head_page_stride;
    if constexpr (DT == DT_BF16) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
        f.k[s] = ld_stream<u32x4>(kp + 1024 * s + 16 * lane);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f.v[j] = ld_stream<u32x2>(vp + ((size_t)(16 * j + n) * kPage + 4 * g) * ES);
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        f.k[s] = ld_stream<u32x4>(kp + ((size_t)n * kHeadDim + 16 * g + 4 * s) * ES);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f.v[j] = ld_stream<u32x4>(vp + ((size_t)(16 * j + n) * kPage + 4 * g) * ES);
    }
  };

  auto compute_page = [&](DecodeFrag<DT>& f, int p) {
    // S^T tile
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == DT_BF16) {
      // LDS operations of one wave run in order, so wavefront-scope fences
      // (compiler ordering only) make the re-deal safe without waits.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
      for (int t = 0; t < 2; ++t) k_lds[w][k_slot(8 * t + (lane >> 3), lane & 7)] = f.k[t];
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < 2; ++t) f.k[t] = k_lds[w][k_slot(n, 4 * t + g)];
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int t = 0; t < 2; ++t)
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, f.k[t]),
                                                    __builtin_bit_cast(bf16x8, qf[t]), s, 0, 0, 0);
    } else {
#pragma unroll
      for (int t = 0; t < 16; ++t)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[t >> 2][t & 3]),
                                                 __uint_as_float(qf[t >> 2][t & 3]), s, 0, 0, 0);
    }
    // tokens 4g + r of this page; mask the tail of the last page
    const int valid = L - (p * kPage + 4 * g);  // tokens of this lane group still < L
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (r < valid) ? s[r] * qk_scale_log2 : kNegInf;
    if (valid < 4) {  // zero V of masked tokens so NaN/Inf junk in the slots cannot leak
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == DT_BF16) {
          unsigned int lo = f.v[j][0], hi = f.v[j][1];
          if (valid < 1) lo &= 0xffff0000u;
          if (valid < 2) lo &= 0x0000ffffu;
          if (valid < 3) hi &= 0xffff0000u;
          hi &= 0x0000ffffu;
          f.v[j][0] = lo;
          f.v[j][1] = hi;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r >= valid) f.v[j][r] = 0u;
        }
      }
    }
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) pv[r] = fast_exp2(x[r] - m_use);
    d_run = d_run * alpha + ((pv[0] + pv[1]) + (pv[2] + pv[3]));
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] *= alpha;
    if constexpr (DT == DT_BF16) {
      const i16x4 pb = __builtin_bit_cast(
          i16x4, u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])});
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, f.v[j]), pb,
                                                         o[j], 0, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          o[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.v[j][r]), pv[r], o[j], 0,
                                                      0, 0);
    }
  };

  // Page walk.  This wave takes pages p_begin + w + WAVES*k, k = 0 .. n_mine-1.
  // Their physical ids are fetched once per 64 pages into one VGPR (lane k
  // holds page k's id) and read back with v_readlane, so the loop never waits
  // on a scalar load.  Page data is double-buffered in registers: the loads
  // of the next UNROLL pages are issued before the current UNROLL pages are
  // consumed, keeping 2*UNROLL pages of this wave in flight.
  const int n_mine = p_end - p_begin - w > 0 ? (p_end - p_begin - w + WAVES - 1) / WAVES : 0;
  int ids = -1;
  auto fetch_ids = [&](int k0) {
    const int k = k0 + lane;
    ids = (k < n_mine) ? pt[p_begin + w + k * WAVES] : -1;
  };
  auto phys_of = [&](int k) { return __builtin_amdgcn_readlane(ids, k & 63); };
  auto load_group = [&](int k0, DecodeFrag<DT>* f, int* ph) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      ph[u] = (k0 + u < n_mine) ? phys_of(k0 + u) : -1;
      if ((unsigned)ph[u] < (unsigned)num_pages) load_page(ph[u], f[u]);
    }
  };
  auto compute_group = [&](int k0, DecodeFrag<DT>* f, const int* ph) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if ((unsigned)ph[u] < (unsigned)num_pages) compute_page(f[u], p_begin + w + (k0 + u) * WAVES);
  };
  static_assert(64 % UNROLL == 0, "page groups must not straddle an id block");
  if (n_mine > 0) {
    DecodeFrag<DT> fa[UNROLL], fb[UNROLL];
    int pa[UNROLL], pb[UNROLL];
    fetch_ids(0);
    load_group(0, fa, pa);
    for (int k = 0; k < n_mine; k += 2 * UNROLL) {
      // ids for the group after next must be resident before it is loaded
      if (((k + UNROLL) & 63) == 0 && k + UNROLL < n_mine) fetch_ids(k + UNROLL);
      if (k + UNROLL < n_mine) load_group(k + UNROLL, fb, pb);
      compute_group(k, fa, pa);
      if (k + UNROLL >= n_mine) break;
      if (((k + 2 * UNROLL) & 63) == 0 && k + 2 * UNROLL < n_mine) fetch_ids(k + 2 * UNROLL);
      if (k + 2 * UNROLL < n_mine) load_group(k + 2 * UNROLL, fa, pa);
      compute_group(k + UNROLL, fb, pb);
    }
  }

  // Combine lane groups, then the waves of the workgroup (same merge rule as
  // the split merge; only one state carries the sink).
  d_run = xor_sum(d_run, 16);
  d_run = xor_sum(d_run, 32);
  __shared__ float sm_m[WAVES][16], sm_d[WAVES][16];
  __shared__ float sm_o[WAVES][16][kHeadDim + 4];
  if (g == 0) {
    sm_m[w][n] = m_run;
    sm_d[w][n] = d_run;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) sm_o[w][n][16 * j + 4 * g + r] = o[j][r];
  __syncthreads();

  for (int idx = threadIdx.x; idx < 16 * 16; idx += 64 * WAVES) {
    const int hh = idx >> 4, d0 = (idx & 15) * 4;
    if (hh >= group) continue;
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) M = fmaxf(M, sm_m[ww][hh]);
    float D = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) {
      const float mw = sm_m[ww][hh];
      const float e = (mw == kNegInf) ? 0.f : fast_exp2(mw - M);
      D += sm_d[ww][hh] * e;
#pragma unroll
      for (int i = 0; i < 4; ++i) O[i] += sm_o[ww][hh][d0 + i] * e;
    }
    const int head = kvh * group + hh;
    const size_t row = (size_t)b * hq + head;
    if (splits == 1) {
      float y[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = D > 0.f ? O[i] / D : 0.f;
      if constexpr (DT == DT_BF16) {
        *reinterpret_cast<u32x2*>(out + (row * kHeadDim + d0) * 2) =
            u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      } else {
        *reinterpret_cast<f32x4*>(out + (row * kHeadDim + d0) * 4) = f32x4{y[0], y[1], y[2], y[3]};
      }
    } else {
      const size_t st = row * splits + c;
      if (d0 == 0) {
        part_m[st] = (M == kNegInf) ? kNegInf : M * kLn2;
        part_d[st] = D;
      }
      *reinterpret_cast<f32x4*>(part_o + st * kHeadDim + d0) = f32x4{O[0], O[1], O[2], O[3]};
    }
  }
}

// ============================================================= merge kernel
//
// CL*16 threads per (sequence, query head) row: thread (cl, dq) owns output
// dims [4dq, 4dq+4) and the chunks c = cl, cl + CL, ...  Every thread issues
// all its loads (m_c, d_c and the 16-byte slice of o_c) before using any, so
// the merge costs one memory round trip; M, then the weights e^(m_c - M),
// the partial sums of d and o, are combined across the CL chunk lanes
// through LDS in a fixed order.

template <int DT, int CL>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ pm,
                                                    const float* __restrict__ pd,
                                                    const float* __restrict__ po, int rows,
                                                    int splits, char* __restrict__ out) {
  constexpr int TPR = 16 * CL;  // threads per row
  constexpr int RPB = 256 / TPR;  // rows per block
  constexpr int MAXC = 8;         // chunks held in registers per thread and pass
  __shared__ float sm_m[RPB][CL];
  __shared__ float sm_d[RPB][CL];
  __shared__ f32x4 sm_o[RPB][CL][16];
  const int t = threadIdx.x % TPR, rl = threadIdx.x / TPR;
  const int row = blockIdx.x * RPB + rl;
  const int cl = t >> 4, dq = t & 15;
  const bool live = row < rows;
  const float* m = pm + (size_t)row * splits;
  const float* d = pd + (size_t)row * splits;
  const float* o = po + (size_t)row * splits * kHeadDim + 4 * dq;

  // The first CL*MAXC chunks (every workload here) are loaded once, all at
  // the same time; chunks beyond that are read in a second, rarely used loop.
  float mv[MAXC], dv[MAXC];
  f32x4 ov[MAXC];
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = cl + i * CL;
    const bool ok = live && c < splits;
    mv[i] = ok ? m[c] : kNegInf;
    dv[i] = ok ? d[c] : 0.f;
    ov[i] = ok ? *reinterpret_cast<const f32x4*>(o + (size_t)c * kHeadDim)
               : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float mloc = kNegInf;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) mloc = fmaxf(mloc, mv[i]);
  for (int c = cl + CL * MAXC; live && c < splits; c += CL) mloc = fmaxf(mloc, m[c]);
  if (dq == 0) sm_m[rl][cl] = mloc;
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < CL; ++k) M = fmaxf(M, sm_m[rl][k]);

  float D = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const float e = (mv[i] == kNegInf) ? 0.f : fast_exp2((mv[i] - M) * kLog2e);
    D += dv[i] * e;
    acc += e * ov[i];
  }
  for (int c = cl + CL * MAXC; live && c < splits; c += CL) {
    const float mc = m[c];
    if (mc == kNegInf) continue;
    const float e = fast_exp2((mc - M) * kLog2e);
    D += d[c] * e;
    acc += e * *reinterpret_cast<const f32x4*>(o + (size_t)c * kHeadDim);
  }
  if (dq == 0) sm_d[rl][cl] = D;
  sm_o[rl][cl][dq] = acc;
  __syncthreads();
  if (cl == 0 && live) {
    f32x4 sum = sm_o[rl][0][dq];
    float Dt = sm_d[rl][0];
#pragma unroll
    for (int k = 1; k < CL; ++k) {
      sum += sm_o[rl][k][dq];
      Dt += sm_d[rl][k];
    }
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = Dt > 0.f ? sum[i] / Dt : 0.f;
    const size_t off = (size_t)row * kHeadDim + 4 * dq;
    if constexpr (DT == DT_BF16) {
      *reinterpret_cast<u32x2*>(out + off * 2) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      *reinterpret_cast<f32x4*>(out + off * 4) = f32x4{y[0], y[1], y[2], y[3]};
    }
  }
}

// =========================================================== prefill kernel
//
// Workgroup = WAVES waves; wave w owns ROWS = 32*RB rows, row r = (token
// r / G, head r % G) of tokens [t_begin + w*TW, +TW), TW = ROWS / G, so every
// query head of a kv group reads the same K/V tile.  Key tiles of 64 are
// staged in LDS: bf16 ragged K/V go from global memory straight into a
// three-stage ring, two tiles ahead of the one in use; paged and fp32 tiles
// pass through registers into a double buffer, one tile ahead.  Per tile
// and wave:
//   S^T[64 keys x ROWS]  = K . Q^T       (2 key blocks x RB row blocks)
//   O^T[64 dims x ROWS] += V^T . P^T     (2 dim blocks x RB row blocks)
// A 32x32 MFMA result gives lane l column l%32 (a row) and the 16 rows
// 8*(r/4) + 4*(l/32) + r%4, r = 0..15 (keys for S^T, dims for O^T).  Each
// row's 64 keys are thus split over lanes l and l^32; its max is one
// cross-lane exchange and its sum is deferred to the end.  The register
// layout of S^T is directly the P^T operand of the next product (same key
// order on the V side), so no shuffle sits between the two products.  bf16
// runs a tile as two staggered 32-key halves (see compute_tile_bf16).

// LDS tiles.  bf16: K and V both row-major with unpadded 128-byte rows,
// XOR-swizzled at 16-byte-chunk granularity (K chunk c of row r at slot
// c ^ (r & 7), V chunk c at slot c ^ 2*(r & 3)); V^T operands are read with
// ds_read_b64_tr_b16.  fp32: K row-major and V transposed (dim-major), rows
// padded by 16 bytes.
template <int DT, int RB, int WAVES>
struct PrefillCfg {
  static constexpr int ES = DT == DT_BF16 ? 2 : 4;
  static constexpr int KROW = kHeadDim + (DT == DT_BF16 ? 0 : 4);  // LDS K row (elements)
  static constexpr int VROW = 64 + (DT == DT_BF16 ? 0 : 4);         // LDS V / Vt row
  static constexpr int NT = 64 * WAVES;
  static constexpr int ROWS = 32 * RB;
  // registers allow 2 waves per SIMD for 64-row bf16 waves, more for 32 rows
  static constexpr int MIN_WAVES_PER_EU = DT == DT_F32 ? 1 : (RB == 2 ? 2 : 3);
};

// Arguments of the prefill kernels.  k / v are either the ragged key / value
// arrays [total_kv, Hkv, D], located per sequence by cu_kv, or (PAGED) the
// caches [pages, Hkv, P, D] / [pages, Hkv, D, P], located by page_table and
// kv_lens.  Without SPLIT the kernel writes out; with SPLIT the key range of
// each sequence is cut into `splits` chunks of whole 16-key units and the
// kernel writes each chunk's partial state (m, d, o) to pm / pd / po.
struct PrefillArgs {
  const char* q;
  const char* k;
  const char* v;
  const float* sinks;
  const int32_t* cu_q;
  const int32_t* cu_kv;
  const int32_t* page_table;
  const int32_t* kv_lens;
  char* out;
  float* pm;
  float* pd;
  float* po;
  int total_q, total_kv, hkv, group, causal, n_qtiles, n_pairs, splits, max_pages, num_pages;
  int rank_seqs;  // map pair ranks to sequences by decreasing query length
  int seq_major;  // with rank_seqs: sequence-major order within each XCD
  uint32_t cache_bytes;  // bytes of each paged cache
  float qk_scale_log2;
};

// Keep the first n elements (16 / es of them) of a 16-byte vector, zero the
// rest: the slots of a sequence's last page past its last key.
__device__ __forceinline__ u32x4 keep_first(u32x4 x, int n, int es) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    unsigned int m;
    if (es == 4)
      m = e < n ? 0xffffffffu : 0u;
    else
      m = 2 * e + 1 < n ? 0xffffffffu : (2 * e < n ? 0x0000ffffu : 0u);
    x[e] &= m;
  }
  return x;
}

// WIDE (paged caches of 4 GiB or more): each page block is read through its
// own buffer resource, built in scalar registers from the block's 64-bit
// address (page ids are wave-uniform), instead of at a 32-bit offset from
// the cache base.
template <int DT, int RB, int WAVES, bool PAGED, bool SPLIT, bool WIDE = false>
__global__ __launch_bounds__(64 * WAVES, (PrefillCfg<DT, RB, WAVES>::MIN_WAVES_PER_EU)) void
prefill_kernel(const PrefillArgs a) {
  static_assert(PAGED || !WIDE, "only paged caches take 64-bit page bases");
  using Cfg = PrefillCfg<DT, RB, WAVES>;
  // Every argument is needed in the prologue: this (pure, so not a memory
  // barrier) empty asm makes them load in one batch here, not in dependent
  // rounds along the branches below.
  int args_ready;
  asm("" : "=s"(args_ready)
      : "s"(a.q), "s"(a.k), "s"(a.v), "s"(a.sinks), "s"(a.cu_q), "s"(a.cu_kv), "s"(a.out),
        "s"(a.total_q), "s"(a.total_kv), "s"(a.hkv), "s"(a.group), "s"(a.n_qtiles), "s"(a.n_pairs),
        "s"(a.rank_seqs), "s"(a.seq_major), "s"(a.qk_scale_log2));
  const char* __restrict__ q = a.q;
  const char* __restrict__ k = a.k;
  const char* __restrict__ v = a.v;
  const float* __restrict__ sinks = a.sinks;
  const int total_q = a.total_q, hkv = a.hkv, group = a.group, causal = a.causal;
  const int n_qtiles = a.n_qtiles, n_pairs = a.n_pairs;
  const float qk_scale_log2 = a.qk_scale_log2;
  constexpr int ES = Cfg::ES, KROW = Cfg::KROW, VROW = Cfg::VROW, NT = Cfg::NT;
  constexpr int BK = 64;  // keys per tile
  // bf16 ragged: three-stage ring filled by direct-to-LDS loads; otherwise
  // two stages filled through registers
  constexpr bool kDma = DT == DT_BF16 && !PAGED;
  static_assert(!kDma || WAVES == 4 || WAVES == 8, "direct-to-LDS staging splits a tile over 4 or 8 waves");
  constexpr int NSTAGE = kDma ? 3 : 2;
  __shared__ __attribute__((aligned(16))) char lds_k[NSTAGE][BK * KROW * ES];
  __shared__ __attribute__((aligned(16))) char lds_v[NSTAGE][kHeadDim * VROW * ES];

  // 1-D grid, (sequence, kv head) pair fastest and query tiles from the last
  // (longest causal key range) to the first: the dispatcher hands out the
  // heaviest work first, and with a pair count that is a multiple of the 8
  // XCDs (workgroups go round-robin over XCDs) every tile of a pair lands on
  // the same XCD, whose L2 then holds that pair's K/V.
  // With SPLIT, the chunks of one query tile are adjacent in dispatch order.
  const int pair = (int)(blockIdx.x % (unsigned)n_pairs);
  int slot = (int)(blockIdx.x / (unsigned)n_pairs);
  int split = SPLIT ? slot % a.splits : 0;
  if constexpr (SPLIT) slot /= a.splits;
  int tile = n_qtiles - 1 - slot;
  int kvh = pair % hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, col = lane & 31;
  const int hq = hkv * group;
  const int TW = Cfg::ROWS / group;  // tokens per wave
  const int TB = WAVES * TW;         // tokens per workgroup

  // For up to 64 sequences of unequal query length the pair's sequence
  // index is read as a rank by decreasing query length (ties by index):
  // within a slot, the workgroups with work are then contiguous and those of
  // sequences too short for the slot's tile (which exit at once) trail them.
  // Interleaved, those empty workgroups skewed the placement of the rest (16
  // ragged sequences: 20% slower).  Every lane loads its own sequence's
  // bounds, so the ranking adds no dependent load.
  //
  // With seq_major (ragged batch and keys, kv heads a multiple of the 8
  // XCDs) the order is instead sequence-major within each XCD: workgroup i
  // runs on XCD i % 8 (workgroups go round-robin over XCDs), which takes kv
  // heads x, x + 8, ... and walks their work items sequence by sequence,
  // longest first, each sequence's query tiles heaviest first (chunks of a
  // tile adjacent).  Only one or two sequences' K/V are then live in an
  // XCD's L2 at a time, where the slot-major order keeps every sequence's
  // live (16 ragged sequences: 8.6 MB of K/V per XCD against a 4 MB L2).
  // Each XCD does the same work; workgroups past an XCD's last item exit.
  const int batch = n_pairs / hkv;
  int b = pair / hkv, q0, q1, k0 = 0, Lkv;
  if (a.rank_seqs) {
    const int bl = min(lane, batch), bh = min(lane + 1, batch);
    const int cq0 = clampi(a.cu_q[bl], 0, total_q), cq1 = clampi(a.cu_q[bh], cq0, total_q);
    int lk0 = 0, lk1;
    if constexpr (PAGED) {
      lk1 = clampi(a.kv_lens[min(lane, batch - 1)], 0, a.max_pages * kPage);
    } else {
      lk0 = clampi(a.cu_kv[bl], 0, a.total_kv);
      lk1 = clampi(a.cu_kv[bh], lk0, a.total_kv);
    }
    const int len = lane < batch ? cq1 - cq0 : -1;
    if (!PAGED && a.seq_major) {
      const int S = SPLIT ? a.splits : 1, hpx = hkv / 8;
      const int j = (int)(blockIdx.x / 8u);
      const int ntq = len > 0 ? (len + TB - 1) / TB : 0;  // query tiles of this lane's sequence
      const int items = ntq * S * hpx;
      // items of the sequences ordered before this lane's (longer, or as
      // long with a lower index)
      int start = 0;
      for (int m = 0; m < batch; ++m) {
        const int lm = __builtin_amdgcn_readlane(len, m), im = __builtin_amdgcn_readlane(items, m);
        start += ((lm > len) || (lm == len && m < lane)) ? im : 0;
      }
      const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < batch && start <= j && j < start + items);
      if (hit == 0) return;
      b = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
      const int local = j - __builtin_amdgcn_readlane(start, b);
      const int per_head = __builtin_amdgcn_readlane(ntq, b) * S;
      kvh = (int)(blockIdx.x % 8u) + 8 * (local / per_head);
      split = (local % per_head) % S;
      tile = __builtin_amdgcn_readlane(ntq, b) - 1 - (local % per_head) / S;
    } else {
      b = nth_longest(len, batch, b);
    }
    q0 = __builtin_amdgcn_readlane(cq0, b);
    q1 = __builtin_amdgcn_readlane(cq1, b);
    k0 = __builtin_amdgcn_readlane(lk0, b);
    Lkv = __builtin_amdgcn_readlane(lk1, b) - k0;
  } else {
    // the sequence's four bounds, loaded together
    const int cq0 = a.cu_q[b], cq1 = a.cu_q[b + 1];
    const int ck0 = PAGED ? 0 : a.cu_kv[b], ck1 = PAGED ? a.kv_lens[b] : a.cu_kv[b + 1];
    asm("" : "=s"(args_ready) : "s"(cq0), "s"(cq1), "s"(ck0), "s"(ck1), "s"(args_ready));
    q0 = clampi(cq0, 0, total_q);
    q1 = clampi(cq1, q0, total_q);
    if constexpr (PAGED) {
      Lkv = clampi(ck1, 0, a.max_pages * kPage);
    } else {
      k0 = clampi(ck0, 0, a.total_kv);
      Lkv = clampi(ck1, k0, a.total_kv) - k0;
    }
  }
  asm volatile("" ::"s"(args_ready));
  const int Lq = q1 - q0;
  const int t_begin = tile * TB;
  if (t_begin >= Lq) return;
  const int t_last = min(t_begin + TB, Lq) - 1;
  const int shift = Lkv - Lq;  // bottom-right causal alignment

  // key chunk [c_lo, c_hi) of this workgroup: ceil(units / splits) whole
  // 16-key units per chunk (page aligned when the keys are paged)
  int c_lo = 0, c_hi = Lkv;
  if constexpr (SPLIT) {
    const int units = (Lkv + kPage - 1) / kPage, per = (units + a.splits - 1) / a.splits;
    c_lo = min(split * per * kPage, Lkv);
    c_hi = min(c_lo + per * kPage, Lkv);
  }

  // keys this workgroup needs, and the key below which no valid row masks
  int n_keys = causal ? min(Lkv, t_last + shift + 1) : Lkv;
  n_keys = min(max(n_keys, 0), c_hi);
  const int n_tiles = n_keys > c_lo ? (n_keys - c_lo + BK - 1) / BK : 0;
  const int lim_min = min(causal ? min(t_begin + shift, Lkv - 1) : Lkv - 1, c_hi - 1);

  // ---- rows of this lane, one per row block
  int lim[RB], head[RB], tok[RB];
  bool valid[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = 32 * rb + col;
    const int tl = r / group, hl = r - tl * group;
    tok[rb] = t_begin + w * TW + tl;
    head[rb] = kvh * group + hl;
    valid[rb] = (tl < TW) && (tok[rb] < Lq);
    lim[rb] = valid[rb] ? min(causal ? min(tok[rb] + shift, Lkv - 1) : Lkv - 1, c_hi - 1) : -1;
  }

  // ---- direct-to-LDS staging (kDma): tile jt goes to stage jt % 3.  Wave w
  // fills key rows 8(w + WAVES u) .. +7 of the K and V tiles (u < 8 / WAVES),
  // 1 KB per load; lane i brings the 16-byte chunk that belongs in slot i % 8 of its
  // row, so the tiles land in the swizzled layouts the operand reads expect
  // (K chunk c at slot c ^ (r & 7), V chunk c at slot c ^ 2(r & 3)).  Keys
  // past the sequence read zero.  The first two tiles are issued before Q.
  u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
  auto dma_issue = [&](int jt) __attribute__((always_inline)) {
    if constexpr (kDma) {
      const uint32_t row_bytes = (uint32_t)hkv * kHeadDim * ES;
      const int key0 = c_lo + jt * BK, stage = jt % NSTAGE;
#pragma unroll
      for (int u = 0; u < 8 / WAVES; ++u) {
        const int key = 8 * (w + WAVES * u) + (lane >> 3), slot = lane & 7;
        const uint32_t row = (uint32_t)(key0 + key) * row_bytes + (uint32_t)kvh * kHeadDim * ES;
        const uint32_t dst = 1024 * (w + WAVES * u);
        load_to_lds16(kw, row + 16 * (slot ^ (key & 7)),
                      __builtin_amdgcn_readfirstlane(lds_addr(lds_k[stage]) + dst));
        load_to_lds16(vw, row + 16 * (slot ^ (2 * (key & 3))),
                      __builtin_amdgcn_readfirstlane(lds_addr(lds_v[stage]) + dst));
      }
    }
  };
  if constexpr (kDma) {
    const uint32_t row_bytes = (uint32_t)hkv * kHeadDim * ES;
    kw = rsrc_words(k + (size_t)k0 * row_bytes, (uint32_t)((size_t)Lkv * row_bytes));
    vw = rsrc_words(v + (size_t)k0 * row_bytes, (uint32_t)((size_t)Lkv * row_bytes));
    if (n_tiles > 0) dma_issue(0);
    if (n_tiles > 1) dma_issue(1);
  }

  // ---- Q^T operand: lane group g owns dims [32g, 32g+32)
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(q + (size_t)q0 * hq * kHeadDim * ES, (uint32_t)((size_t)Lq * hq * kHeadDim * ES));
  constexpr int QV = DT == DT_BF16 ? 4 : 8;  // 16-byte vectors per lane per row
  u32x4 qf[RB][QV];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint32_t base = ((uint32_t)tok[rb] * hq + head[rb]) * kHeadDim * ES + 32 * g * ES;
#pragma unroll
    for (int s = 0; s < QV; ++s)
      qf[rb][s] = valid[rb] ? buf_load16(qr, base + 16 * s) : u32x4{0, 0, 0, 0};
  }

  // ---- running state per row (log2 units), starting from the sink: m = s,
  // d = e^(s - m) = 1 (0 for s = -inf), counted in lane group 0 only because
  // d is summed over the two lanes of a row at the end.  Of a split key
  // range only the first chunk carries the sink; the others start empty.
  float m_run[RB], d_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float s = (valid[rb] && split == 0) ? sinks[head[rb]] : kNegInf;
    // rows past the tile's tokens get a finite reference: their (unused) P
    // then never asks for the slow path
    m_run[rb] = valid[rb] ? s * kLog2e : 0.f;
    d_run[rb] = (g == 0 && s != kNegInf) ? 1.f : 0.f;
  }
  f32x16 acc_o[2][RB];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc_o[db][rb][i] = 0.f;

  // ---- K/V staging of paged and fp32 tiles: global (buffer loads, zero past
  // the sequence) -> registers -> LDS, one tile ahead
  const uint32_t kv_row_bytes = (uint32_t)hkv * kHeadDim * ES;
  const __amdgpu_buffer_rsrc_t kr =
      PAGED ? make_rsrc(k, a.cache_bytes)
            : make_rsrc(k + (size_t)k0 * kv_row_bytes, (uint32_t)((size_t)Lkv * kv_row_bytes));
  const __amdgpu_buffer_rsrc_t vr =
      PAGED ? make_rsrc(v, a.cache_bytes)
            : make_rsrc(v + (size_t)k0 * kv_row_bytes, (uint32_t)((size_t)Lkv * kv_row_bytes));
  constexpr int CPR = kHeadDim * ES / 16;             // 16-byte chunks per key row
  constexpr int NCH = (BK * CPR + NT - 1) / NT;       // K chunks per thread
  constexpr int VITEMS = BK * CPR;                    // V chunks (one key row each)
  constexpr int NCV = (VITEMS + NT - 1) / NT;
  constexpr int VREG = 1;
  u32x4 stk[NCH], stv[NCV][VREG];
  const uint32_t head_off = (uint32_t)kvh * kHeadDim * ES;

  // Paged: a tile of 64 keys is 4 whole pages (chunks start on a page).  A
  // (page, kv head) block of either cache is 16 * 64 elements, contiguous,
  // and chunk c of a tile is its 16-byte piece c % (16 CPR) -- a key row
  // piece for K, a dim row piece for the dim-major V -- in page c / (16 CPR)
  // of the tile.  A wave's 64 consecutive chunks share one page, so page ids
  // and page base offsets are wave-uniform.  The ids are fetched one tile
  // ahead with vector loads (which complete in order with the data loads, so
  // no wait in the tile's compute is held up by them) and moved to scalar
  // registers only when the next tile's loads are issued.
  static_assert(NCV == NCH, "K and V chunks of a tile must pair up");
  static_assert((kPage * CPR) % 64 == 0, "a wave's chunks must share a page");
  const __amdgpu_buffer_rsrc_t ptr =
      make_rsrc(PAGED ? a.page_table + (size_t)b * a.max_pages : nullptr,
                PAGED ? (uint32_t)a.max_pages * 4u : 0u);
  int pid_next[NCH];
  auto page_of = [&](int jt, int u) {
    return (c_lo + jt * BK) / kPage + (64 * w + NT * u) / (kPage * CPR);
  };
  auto fetch_ids = [&](int jt) {
    if constexpr (PAGED) {
#pragma unroll
      for (int u = 0; u < NCH; ++u)
        pid_next[u] = __builtin_amdgcn_raw_buffer_load_b32(ptr, 0, 4 * page_of(jt, u), 0);
    }
  };

  auto stage_load = [&](int jt) {
    const int key0 = c_lo + jt * BK;
    if constexpr (PAGED) {
      constexpr uint32_t kBlock = kPage * kHeadDim * ES;  // one (page, kv head) block
      // all ids to scalar registers first: the wait for them then comes
      // before this tile's data loads are issued, not after
      int ids[NCH];
#pragma unroll
      for (int u = 0; u < NCH; ++u) ids[u] = __builtin_amdgcn_readfirstlane(pid_next[u]);
#pragma unroll
      for (int u = 0; u < NCH; ++u) {
        const int c = tid + NT * u;
        const int vrem = c % (kPage * CPR);
        const int tp = (64 * w + NT * u) / (kPage * CPR);  // page of the tile (uniform)
        const int id = ids[u];
        // pages past the sequence and bad ids (outside [0, num_pages)) are skipped
        if (page_of(jt, u) * kPage < Lkv && id >= 0 && id < a.num_pages) {
          if constexpr (WIDE) {
            // one buffer resource per page block, built in scalar registers
            const size_t base = ((size_t)id * hkv + kvh) * kBlock;
            stk[u] = buf_load16(make_rsrc(k + base, kBlock), 16 * vrem);
            stv[u][0] = buf_load16(make_rsrc(v + base, kBlock), 16 * vrem);
          } else {
            const uint32_t base = ((uint32_t)id * hkv + kvh) * kBlock;
            stk[u] = buf_load16(kr, 16 * vrem, base);
            stv[u][0] = buf_load16(vr, 16 * vrem, base);
          }
          // slots of the sequence's last page past its last key: zero V (their
          // scores are masked, and 0 * junk must not reach O)
          if (key0 + (tp + 1) * kPage > Lkv)
            stv[u][0] = keep_first(stv[u][0], Lkv - (key0 + tp * kPage + (vrem % ES) * (16 / ES)),
                                   ES);
        } else {
          stk[u] = u32x4{0, 0, 0, 0};
          stv[u][0] = u32x4{0, 0, 0, 0};
        }
      }
      fetch_ids(jt + 1);
      return;
    }
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + NT * u, key = c / CPR, part = c % CPR;
      if (c < BK * CPR)
        stk[u] = buf_load16(kr, (uint32_t)(key0 + key) * kv_row_bytes + head_off + part * 16);
    }
#pragma unroll
    for (int u = 0; u < NCV; ++u) {
      const int c = tid + NT * u, part = c % CPR;
      if (c < VITEMS) {
#pragma unroll
        for (int x = 0; x < VREG; ++x) {
          const int key = (c / CPR) * VREG + x;
          stv[u][x] = buf_load16(vr, (uint32_t)(key0 + key) * kv_row_bytes + head_off + part * 16);
        }
      }
    }
  };

  auto stage_store = [&](int buf) {
    char* kd = lds_k[buf];
    char* vd = lds_v[buf];
#pragma unroll
    for (int u = 0; u < NCH; ++u) {
      const int c = tid + NT * u, key = c / CPR, part = c % CPR;
      if (c < BK * CPR) {
        if constexpr (DT == DT_BF16)
          *reinterpret_cast<u32x4*>(kd + key * 128 + 16 * (part ^ (key & 7))) = stk[u];
        else
          *reinterpret_cast<u32x4*>(kd + (key * KROW + part * (16 / ES)) * ES) = stk[u];
      }
    }
    if constexpr (PAGED) {
      // V^T tile [64 dims][64 keys].  bf16: a 128-byte dim row holds 8 pairs
      // of 4-key granules; pair 2m + r (r = 0, 1) of the 16-key group m is
      // granules 4m + r and 4m + r + 2, which is exactly what one lane's P.V
      // operand needs, so it reads one 16-byte pair.  Pair p of row d sits
      // at slot p ^ ((d >> 1) & 7): the 16 rows of a read phase hit distinct
      // banks.  A staged chunk (8 keys of one dim row, page tp of the tile,
      // half vp) fills half vp of pairs 2tp and 2tp + 1.  fp32: rows padded
      // by 16 bytes.
#pragma unroll
      for (int u = 0; u < NCV; ++u) {
        const int c = tid + NT * u;
        if (c >= VITEMS) continue;
        const int vrem = c % (kPage * CPR), dim = vrem / ES, vp = vrem % ES;
        const int tp = c / (kPage * CPR);
        const u32x4 x = stv[u][0];
        if constexpr (DT == DT_BF16) {
          const int sw = (dim >> 1) & 7;
          char* row = vd + dim * 128 + 8 * vp;
          *reinterpret_cast<u32x2*>(row + 16 * ((2 * tp) ^ sw)) = u32x2{x[0], x[1]};
          *reinterpret_cast<u32x2*>(row + 16 * ((2 * tp + 1) ^ sw)) = u32x2{x[2], x[3]};
        } else {
          *reinterpret_cast<u32x4*>(vd + (dim * VROW + tp * kPage + 4 * vp) * ES) = x;
        }
      }
      return;
    }
    // fp32 ragged V, transposed to dim-major (bf16 ragged tiles are loaded
    // straight into LDS and never come here)
#pragma unroll
    for (int u = 0; u < NCV; ++u) {
      const int c = tid + NT * u, part = c % CPR, key = c / CPR;
      if (c >= VITEMS) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<unsigned int*>(vd + ((4 * part + i) * VROW + key) * ES) = stv[u][0][i];
    }
  };

  // fp32 (the instance behind the 1e-5 parity tests): the whole 64-key tile
  // in one pass on v_mfma_f32_32x32x2f32, P kept in fp32.
  auto compute_tile_f32 = [&](auto masked, int buf, int jt) {
    const char* kd = lds_k[buf];
    const char* vd = lds_v[buf];
    f32x16 sacc[2][RB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][rb][i] = 0.f;

    // S^T = K Q^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const char* krow = kd + ((kb * 32 + col) * KROW + 32 * g) * ES;
#pragma unroll
      for (int s = 0; s < QV; ++s) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 16 * s);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            sacc[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                __uint_as_float(kf[e]), __uint_as_float(qf[rb][s][e]), sacc[kb][rb], 0, 0, 0);
      }
    }

    // Online softmax against a lazily kept reference m_run (log2 units) that
    // starts at the sink.  P = 2^(x - m_run) is formed directly, with no row
    // max per tile: the reference only has to keep P finite and bounded, and
    // O/d does not depend on which reference is used.  A row takes the slow
    // path -- true max of the tile, rescale of its O and d, P formed again --
    // when it has no reference yet (m_run = -inf) or when a lane's share of
    // the tile's row sum exceeds kLaneSumMax (which also catches an
    // infinite P).  The branch is wave-uniform, but only the rows that need
    // it change, so a row's result never depends on other rows.
    float pt[RB][2][16];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (decltype(masked)::value) {
        // key = c_lo + jt*BK + kb*32 + 4g + off(r), off(r) = 8*(r/4) + r%4 a
        // constant: compare off(r) with one per-lane threshold per key block
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int thr = lim[rb] - (c_lo + jt * BK + kb * 32 + 4 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][rb][r] = (8 * (r >> 2) + (r & 3) > thr) ? kNegInf : sacc[kb][rb][r];
        }
      }
      // P of this row block against reference m; returns the lane's row sum
      auto form_p = [&](float m) {
        const float m_use = (m == kNegInf) ? 0.f : m;
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float pr = fast_exp2(__builtin_fmaf(sacc[kb][rb][r], qk_scale_log2, -m_use));
            pt[rb][kb][r] = pr;
            ps[r & 3] += pr;
          }
        return (ps[0] + ps[1]) + (ps[2] + ps[3]);
      };
      float rs = form_p(m_run[rb]);
      const bool slow = !(rs <= kLaneSumMax) || m_run[rb] == kNegInf;
      if (wave_any(slow)) {
        // rows (both lanes) that need a new reference move it to the max of
        // their reference and this tile's logits; the others keep theirs and
        // form bit-identical P again
        const bool need = xor_max(slow ? 1.f : 0.f, 32) > 0.f;
        float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            float& a = mx4[(kb * 8 + r / 2) & 3];
            a = fmaxf(fmaxf(a, sacc[kb][rb][r]), sacc[kb][rb][r + 1]);
          }
        const float mx =
            xor_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])), 32) * qk_scale_log2;
        const float m_new = need ? fmaxf(m_run[rb], mx) : m_run[rb];
        const float alpha = (m_new == m_run[rb]) ? 1.f : fast_exp2(m_run[rb] - m_new);
        d_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db) acc_o[db][rb] *= alpha;
        m_run[rb] = m_new;
        rs = form_p(m_new);
      }
      d_run[rb] += rs;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const char* vrow = vd + ((db * 32 + col) * VROW) * ES;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const u32x4 vf = *reinterpret_cast<const u32x4*>(vrow + (kb * 32 + 8 * qd + 4 * g) * ES);
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc_o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                  __uint_as_float(vf[e]), pt[rb][kb][4 * qd + e], acc_o[db][rb], 0, 0, 0);
        }
    }
  };

  // Per-lane byte offsets of the bf16 MFMA operands inside a stage.  Key
  // blocks, key steps and dim blocks then differ by constants that the LDS
  // reads take as immediate offsets, so a tile adds its stage base once per
  // offset.  The XOR swizzles only see bits that those constants leave alone.
  //  K, k-step s (key block kb: +4096): row col, chunk (4g + s) ^ (col & 7).
  //  V ragged, dim block db (key rows +32kb +16hh, second half +8 rows):
  //    rows 4g + sl/4, chunk ((32db + 16((lane>>4)&1) + 4(sl&3)) >> 3) ^
  //    2((sl/4)&3), byte 8(sl&1) of it, sl = lane % 16 (the transposing read
  //    hands lane i element i of four 4-element rows).
  //  V paged, key step t = 2kb + hh (dim block db: +4096): dim row col, pair
  //    (2t + g) ^ ((col >> 1) & 7).
  int k_off[4], v_off[PAGED ? 4 : 2];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) k_off[s4] = col * 128 + 16 * ((4 * g + s4) ^ (col & 7));
  if constexpr (PAGED) {
#pragma unroll
    for (int t = 0; t < 4; ++t) v_off[t] = col * 128 + 16 * ((2 * t + g) ^ ((col >> 1) & 7));
  } else {
    const int sl = lane & 15;
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      const int chunk = (32 * db + 16 * ((lane >> 4) & 1) + 4 * (sl & 3)) >> 3;
      v_off[db] = (4 * g + (sl >> 2)) * 128 + 16 * (chunk ^ (2 * ((sl >> 2) & 3))) + 8 * (sl & 1);
    }
  }

  // bf16: the tile runs as two halves of 32 keys (kb = 0, 1) whose products
  // and softmax are staggered -- S^T of half 1 beside the softmax of half 0,
  // O^T += V^T P^T of half 0 beside the softmax of half 1 -- so that every
  // wave has MFMA and VALU work in the same instruction window.  The halves
  // read disjoint K and V operands, so no operand stays live across them.
  // Each half takes the reference check of the full-tile body on its own.
  auto compute_tile_bf16 = [&](auto masked, int buf, int jt) __attribute__((always_inline)) {
    const char* kd = lds_k[buf];
    const char* vd = lds_v[buf];
    f32x16 sacc[2][RB];
    u32x4 pf[RB][2][2];  // P^T operands [rb][kb][hh]
    // This stage's operand addresses: stage base + lane offset, one add each
    // per tile; the empty asm keeps the sums opaque so that the constants
    // below stay immediate offsets of the LDS reads.
    typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds_addr(kd));
    const uint32_t vbase = __builtin_amdgcn_readfirstlane(lds_addr(vd));
    uint32_t ka[4], va[PAGED ? 4 : 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i] = kbase + (uint32_t)k_off[i];
      asm volatile("" : "+v"(ka[i]));
    }
#pragma unroll
    for (int i = 0; i < (PAGED ? 4 : 2); ++i) {
      va[i] = vbase + (uint32_t)v_off[i];
      asm volatile("" : "+v"(va[i]));
    }
    // K operand of k-step s, key block kb: key row 32kb + col, chunk 4g + s
    auto k_operand = [&](int s, int kb) __attribute__((always_inline)) {
      return *(lds_u32x4*)(size_t)(ka[s] + kb * 4096);
    };
    // V^T operand of dim block db for key step (kb, hh)
    auto v_operand = [&](int kb, int hh, int db) __attribute__((always_inline)) {
      if constexpr (PAGED) {
        return *(lds_u32x4*)(size_t)(va[2 * kb + hh] + db * 4096);
      } else {
        // key rows r0 = 32kb + 16hh + 4g + sl/4 and r0 + 8
        const uint32_t p = va[db] + (32 * kb + 16 * hh) * 128;
        const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)p);
        const i16x4 c =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(size_t)(p + 8 * 128));
        const u32x2 lo = __builtin_bit_cast(u32x2, a), hi = __builtin_bit_cast(u32x2, c);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    // S^T of half kb: 4 k-steps x RB MFMAs, K operands of step s + 1 read
    // before the MFMAs of step s
    auto qk = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][rb][i] = 0.f;
      u32x4 kf[2];
      kf[0] = k_operand(0, kb);
#pragma unroll
      for (int s = 0; s < QV; ++s) {
        if (s + 1 < QV) kf[(s + 1) & 1] = k_operand(s + 1, kb);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          sacc[kb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf[s & 1]), __builtin_bit_cast(bf16x8, qf[rb][s]),
              sacc[kb][rb], 0, 0, 0);
      }
    };
    auto mask = [&](int kb) __attribute__((always_inline)) {
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int thr = lim[rb] - (c_lo + jt * BK + kb * 32 + 4 * g);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][rb][r] = (8 * (r >> 2) + (r & 3) > thr) ? kNegInf : sacc[kb][rb][r];
        }
      }
    };
    // P of (half kb, row block rb) against reference m; returns the lane's
    // share of the row sum (the reference-check path)
    auto form_p = [&](int kb, int rb, float m) __attribute__((always_inline)) {
      const float m_use = (m == kNegInf) ? 0.f : m;
      float ps[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * hh + 2 * e;
          const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][rb][r], qk_scale_log2, -m_use));
          const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][rb][r + 1], qk_scale_log2, -m_use));
          pf[rb][kb][hh][e] = pack_bf16x2(p0, p1);
          ps[e] = hh == 0 ? p0 + p1 : ps[e] + (p0 + p1);
        }
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    };
    // Common path, one logit pair at a time: pair q = 0..15 of half kb is
    // row block q / 8, key step (q / 4) % 2, register pair q % 4.
    float mneg[RB], ps[RB][4], rs[RB];
    bool slow[RB];
    // A slot's two pairs are exponentiated in that slot and packed and
    // summed in the next one, so the exponentials' latency is spent under
    // the next MFMA rather than waited on.
    auto pair_exp = [&](int kb, int q, float* ex) __attribute__((always_inline)) {
      const int rb = q >> 3, hh = (q >> 2) & 1, e = q & 3, r = 8 * hh + 2 * e;
      ex[0] = fast_exp2(__builtin_fmaf(sacc[kb][rb][r], qk_scale_log2, mneg[rb]));
      ex[1] = fast_exp2(__builtin_fmaf(sacc[kb][rb][r + 1], qk_scale_log2, mneg[rb]));
    };
    auto pair_fin = [&](int kb, int q, const float* ex) __attribute__((always_inline)) {
      const int rb = q >> 3, hh = (q >> 2) & 1, e = q & 3;
      pf[rb][kb][hh][e] = pack_bf16x2(ex[0], ex[1]);
      ps[rb][e] = hh == 0 ? ex[0] + ex[1] : ps[rb][e] + (ex[0] + ex[1]);
    };
    float ex[2][4];  // exponentials of the last two slots' pairs
    auto start_half = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mneg[rb] = m_run[rb] == kNegInf ? 0.f : -m_run[rb];
    };
    // row sums, the reference check (one wave-uniform branch per half, so
    // the common path of both row blocks stays ahead of it) and d
    auto end_half = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        rs[rb] = (ps[rb][0] + ps[rb][1]) + (ps[rb][2] + ps[rb][3]);
        slow[rb] = !(rs[rb] <= kLaneSumMax) || m_run[rb] == kNegInf;
      }
      if (wave_any(slow[0] || slow[RB - 1])) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          if (!wave_any(slow[rb])) continue;
          const bool need = xor_max(slow[rb] ? 1.f : 0.f, 32) > 0.f;
          float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
          for (int r = 0; r < 16; r += 2)
            mx4[(r / 2) & 3] = fmaxf(fmaxf(mx4[(r / 2) & 3], sacc[kb][rb][r]), sacc[kb][rb][r + 1]);
          const float mx =
              xor_max(fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3])), 32) * qk_scale_log2;
          const float m_new = need ? fmaxf(m_run[rb], mx) : m_run[rb];
          const float alpha = (m_new == m_run[rb]) ? 1.f : fast_exp2(m_run[rb] - m_new);
          d_run[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db) acc_o[db][rb] *= alpha;
          m_run[rb] = m_new;
          rs[rb] = form_p(kb, rb, m_new);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) d_run[rb] += rs[rb];
    };
    static_assert(RB == 2, "the staggered schedule pairs two row blocks");
    // scheduling fence: instructions are not moved across it
#define ATTN_SINK_FENCE() __builtin_amdgcn_sched_barrier(0)
    // S^T of half 0, with the first K operand of half 1 read early
    qk(0);
    u32x4 kf[2];
    kf[0] = k_operand(0, 1);
    mask(0);
    start_half();
    ATTN_SINK_FENCE();
    // S^T of half 1: each MFMA followed by two logit pairs of half 0
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[1][rb][i] = 0.f;
#pragma unroll
    for (int s = 0; s < QV; ++s) {
      if (s + 1 < QV) kf[(s + 1) & 1] = k_operand(s + 1, 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        sacc[1][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, kf[s & 1]), __builtin_bit_cast(bf16x8, qf[rb][s]),
            sacc[1][rb], 0, 0, 0);
        ATTN_SINK_FENCE();
        const int j = 2 * s + rb;
        pair_exp(0, 2 * j, &ex[j & 1][0]);
        pair_exp(0, 2 * j + 1, &ex[j & 1][2]);
        if (j > 0) {
          pair_fin(0, 2 * j - 2, &ex[(j - 1) & 1][0]);
          pair_fin(0, 2 * j - 1, &ex[(j - 1) & 1][2]);
        }
        ATTN_SINK_FENCE();
      }
    }
    pair_fin(0, 14, &ex[1][0]);
    pair_fin(0, 15, &ex[1][2]);
    end_half(0);
    // O^T += V^T P^T of half 0: each MFMA followed by two logit pairs of half
    // 1; the four slots of its second key step also read the V operands of
    // half 1 (vg[hh][db]), so that their LDS latency is hidden there
    mask(1);
    start_half();
    u32x4 vf[2][2], vg[2][2];
    vf[0][0] = v_operand(0, 0, 0);
    vf[0][1] = v_operand(0, 0, 1);
    vf[1][0] = v_operand(0, 1, 0);
    vf[1][1] = v_operand(0, 1, 1);
    ATTN_SINK_FENCE();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc_o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, vf[hh][db]), __builtin_bit_cast(bf16x8, pf[rb][0][hh]),
              acc_o[db][rb], 0, 0, 0);
          ATTN_SINK_FENCE();
          const int j = 4 * hh + 2 * db + rb;
          pair_exp(1, 2 * j, &ex[j & 1][0]);
          pair_exp(1, 2 * j + 1, &ex[j & 1][2]);
          if (j > 0) {
            pair_fin(1, 2 * j - 2, &ex[(j - 1) & 1][0]);
            pair_fin(1, 2 * j - 1, &ex[(j - 1) & 1][2]);
          }
          if (hh == 1) vg[db][rb] = v_operand(1, db, rb);  // (db, rb) as (hh, db)
          ATTN_SINK_FENCE();
        }
    pair_fin(1, 14, &ex[1][0]);
    pair_fin(1, 15, &ex[1][2]);
    end_half(1);
    // O^T += V^T P^T of half 1
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
          acc_o[db][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, vg[hh][db]), __builtin_bit_cast(bf16x8, pf[rb][1][hh]),
              acc_o[db][rb], 0, 0, 0);
#undef ATTN_SINK_FENCE
  };

  // Tiles below n_plain need no mask for any valid row of the workgroup; the
  // remaining (diagonal / ragged-tail) tiles run the masked body.  Two loops
  // keep the mask arithmetic out of the common path.
  const int n_plain = min(n_tiles, max(0, (lim_min + 1 - c_lo) / BK));
  if constexpr (kDma) {
    // Q and the first two tiles were issued together: wait for all of them
    // (a wait the compiler sees, so it adds none for Q later), then per tile
    // issue tile jt + 2, compute tile jt, wait until only tile jt + 2's four
    // loads are outstanding (tile jt + 1 has landed), and barrier.  The
    // barrier also frees stage jt % 3 for tile jt + 3.
    auto tile_step = [&](auto masked, int jt) __attribute__((always_inline)) {
      if (jt + 2 < n_tiles) dma_issue(jt + 2);
      compute_tile_bf16(masked, jt % NSTAGE, jt);
      // tile jt + 2's loads (2 * 8 / WAVES per wave) may stay in flight
      if (jt + 2 < n_tiles) {
        if constexpr (WAVES == 4)
          asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        else
          asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      lds_barrier();
    };
    if (n_tiles > 0) {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      lds_barrier();
      int jt = 0;
      for (; jt < n_plain; ++jt) tile_step(std::false_type{}, jt);
      for (; jt < n_tiles; ++jt) tile_step(std::true_type{}, jt);
    }
  } else if (n_tiles > 0) {
    fetch_ids(0);
    stage_load(0);
    stage_store(0);
    __syncthreads();
    int jt = 0;
    for (; jt < n_plain; ++jt) {
      const bool more = jt + 1 < n_tiles;
      if (more) stage_load(jt + 1);
      if constexpr (DT == DT_BF16)
        compute_tile_bf16(std::false_type{}, jt & 1, jt);
      else
        compute_tile_f32(std::false_type{}, jt & 1, jt);
      if (more) stage_store((jt + 1) & 1);
      __syncthreads();
    }
    for (; jt < n_tiles; ++jt) {
      const bool more = jt + 1 < n_tiles;
      if (more) stage_load(jt + 1);
      if constexpr (DT == DT_BF16)
        compute_tile_bf16(std::true_type{}, jt & 1, jt);
      else
        compute_tile_f32(std::true_type{}, jt & 1, jt);
      if (more) stage_store((jt + 1) & 1);
      __syncthreads();
    }
  }

  // ---- epilogue, bf16 output: the wave's 64 x 64 tile of O / d goes through
  // 8 KB of the (now idle) staging LDS, so that each store writes 8 whole
  // 128-byte rows (1 KB contiguous when the group is 8 heads of one token):
  // stored straight from the MFMA layout, every store instruction touched 64
  // rows 8 bytes at a time.  In LDS, 16-byte chunk c of row r sits at slot
  // c ^ (r & 7).
  constexpr bool kLdsEpilogue = DT == DT_BF16 && !SPLIT && WAVES <= 2 * NSTAGE &&
                                BK * KROW * ES >= 8192 && kHeadDim * VROW * ES >= 8192;
  if constexpr (kLdsEpilogue) {
    char* ob = w < NSTAGE ? lds_k[w] : lds_v[w - NSTAGE];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float dsum = xor_sum(d_run[rb], 32);
      const float inv = dsum > 0.f ? 1.f / dsum : 0.f;
      const int r = 32 * rb + col;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const int c = 4 * db + qd;  // dims 8c + 4g + 0..3
          const float y0 = acc_o[db][rb][4 * qd + 0] * inv, y1 = acc_o[db][rb][4 * qd + 1] * inv;
          const float y2 = acc_o[db][rb][4 * qd + 2] * inv, y3 = acc_o[db][rb][4 * qd + 3] * inv;
          *reinterpret_cast<u32x2*>(ob + r * 128 + 16 * (c ^ (r & 7)) + 8 * g) =
              u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int c = lane & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * i + (lane >> 3);
      const u32x4 x = *reinterpret_cast<const u32x4*>(ob + r * 128 + 16 * (c ^ (r & 7)));
      const int tl = r / group, hl = r - tl * group;
      const int t = t_begin + w * TW + tl;
      if (tl < TW && t < Lq)
        *reinterpret_cast<u32x4*>(a.out + (((size_t)q0 + t) * hq + kvh * group + hl) * kHeadDim * ES +
                                  16 * c) = x;
    }
    return;
  }

  // ---- epilogue: out = O / d (SPLIT: the state m, d, O of this chunk, m in
  // natural-log units), rows of this lane, dims 32db + 8qd + 4g + 0..3
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float dsum = xor_sum(d_run[rb], 32);
    if (!valid[rb]) continue;
    if constexpr (SPLIT) {
      const size_t st = (((size_t)q0 + tok[rb]) * hq + head[rb]) * a.splits + split;
      if (g == 0) {
        a.pm[st] = m_run[rb] * kLn2;
        a.pd[st] = dsum;
      }
      float* po = a.po + st * kHeadDim;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *reinterpret_cast<f32x4*>(po + 32 * db + 8 * qd + 4 * g) =
              f32x4{acc_o[db][rb][4 * qd + 0], acc_o[db][rb][4 * qd + 1],
                    acc_o[db][rb][4 * qd + 2], acc_o[db][rb][4 * qd + 3]};
      continue;
    }
    const float inv = dsum > 0.f ? 1.f / dsum : 0.f;
    char* orow = a.out + (((size_t)q0 + tok[rb]) * hq + head[rb]) * kHeadDim * ES;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * db + 8 * qd + 4 * g;
        const float y0 = acc_o[db][rb][4 * qd + 0] * inv, y1 = acc_o[db][rb][4 * qd + 1] * inv;
        const float y2 = acc_o[db][rb][4 * qd + 2] * inv, y3 = acc_o[db][rb][4 * qd + 3] * inv;
        if constexpr (DT == DT_BF16) {
          *reinterpret_cast<u32x2*>(orow + d0 * ES) = u32x2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
        } else {
          *reinterpret_cast<f32x4*>(orow + d0 * ES) = f32x4{y0, y1, y2, y3};
        }
      }
  }
}

// ============================================================= host side

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool finite_positive(float x) { return x > 0.f && x < __builtin_huge_valf(); }

int launch_status() {
  return hipGetLastError() == hipSuccess ? ATTN_SINK_OK : ATTN_SINK_ERR_LAUNCH;
}

// bf16 prefill: waves of 64 rows per workgroup.
#ifndef ATTN_SINK_PREFILL_WAVES
#define ATTN_SINK_PREFILL_WAVES 4
#endif
constexpr int kPrefillWaves = ATTN_SINK_PREFILL_WAVES;

// Split decode workgroup shape: waves per workgroup and pages per register
// group (two groups are in flight per wave).  Eight waves (two workgroups per
// CU at 128 VGPRs): the B = 64 mixed-length decode at 3 splits + merge runs
// 102.7-103.1 us against 104.5-105.4 with four waves.
#ifndef ATTN_SINK_DECODE_WAVES
#define ATTN_SINK_DECODE_WAVES 8
#endif
#ifndef ATTN_SINK_DECODE_UNROLL
#define ATTN_SINK_DECODE_UNROLL 2
#endif
constexpr int kDecodeWaves = ATTN_SINK_DECODE_WAVES;
constexpr int kDecodeUnroll = ATTN_SINK_DECODE_UNROLL;
// Unsplit decode (one chunk per sequence and kv head): 16 waves per
// workgroup (one workgroup per CU at 128 VGPRs and 104 KB of LDS) split the
// chunk's pages 16 ways and merge in LDS -- a split and its merge in a
// single launch, with no partial state leaving the CU.  Splits across
// workgroups would need a device-wide release between two XCDs' L2s to
// merge in the same launch; 16 waves per workgroup instead cut the
// unsplit decode of the B = 64 mixed-length workload from 117 to 107 us.
#ifndef ATTN_SINK_DECODE_WAVES_UNSPLIT
#define ATTN_SINK_DECODE_WAVES_UNSPLIT 16
#endif
constexpr int kDecodeWavesUnsplit = ATTN_SINK_DECODE_WAVES_UNSPLIT;

// Launch the prefill kernel for (dtype, key source, output form): a 1-D grid
// of query tiles x (sequence, kv head) pairs x key chunks.
template <bool PAGED, bool SPLIT, bool WIDE = false>
int launch_prefill(PrefillArgs a, int dtype, int batch, int max_seqlen_q, hipStream_t s) {
  if ((int64_t)batch * a.hkv > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;
  a.n_pairs = batch * a.hkv;
  const int waves = dtype == ATTN_SINK_BF16 ? kPrefillWaves : 4;
  const int tb = waves * (64 / a.group);  // waves of 64 rows
  a.n_qtiles = (max_seqlen_q + tb - 1) / tb;
  // With every query length equal to max_seqlen_q no slot has empty
  // workgroups, and the ranking would only lengthen the prologue.
  a.rank_seqs = batch <= 64 && (int64_t)batch * max_seqlen_q != (int64_t)a.total_q;
  // (ragged keys only: the paged kernels sit at the register limit, and the
  // extra prologue code cost them 1%)
  a.seq_major = !PAGED && a.rank_seqs && a.hkv % 8 == 0;
  const int64_t blocks = (int64_t)a.n_qtiles * a.n_pairs * (SPLIT ? a.splits : 1);
  if (blocks > INT32_MAX) return ATTN_SINK_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)blocks);
  if (dtype == ATTN_SINK_F32)
    hipLaunchKernelGGL((prefill_kernel<DT_F32, 2, 4, PAGED, SPLIT, WIDE>), grid, dim3(256), 0, s,
                       a);
  else
    hipLaunchKernelGGL((prefill_kernel<DT_BF16, 2, kPrefillWaves, PAGED, SPLIT, WIDE>), grid,
                       dim3(64 * kPrefillWaves), 0, s, a);
  return launch_status();
}

// Checks shared by the prefill entry points (query side and scalars).
int check_prefill_common(const void* q, const float* sinks, const int32_t* cu_seqlens_q,
                         int batch, int total_q, int max_seqlen_q, int num_kv_heads,
                         int group_size, int head_dim, float sm_scale, int causal, int dtype) {
  if (!sinks || !cu_seqlens_q || (!q && total_q != 0)) return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(sinks, 4) || !aligned(cu_seqlens_q, 4))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (batch < 0 || total_q < 0 || max_seqlen_q < 0 || num_kv_heads < 1 || group_size < 1 ||
      head_dim < 1 || (causal != 0 && causal != 1) ||
      (dtype != ATTN_SINK_F32 && dtype != ATTN_SINK_BF16) || !finite_positive(sm_scale))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || group_size > 64) return ATTN_SINK_ERR_UNSUPPORTED;
  const int es = dtype == ATTN_SINK_BF16 ? 2 : 4;
  // buffer offsets are 32-bit: each whole tensor must stay below 4 GiB
  if ((int64_t)total_q * num_kv_heads * group_size * kHeadDim * es >= (int64_t)1 << 32)
    return ATTN_SINK_ERR_UNSUPPORTED;
  return ATTN_SINK_OK;
}

// Checks of the split-KV partial outputs of a prefill entry point.
int check_partials(int num_splits, const float* pm, const float* pd, const float* po) {
  if (num_splits < 1 || num_splits > 65536) return ATTN_SINK_ERR_INVALID_ARG;
  if (!pm || !pd || !po) return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(pm, 4) || !aligned(pd, 4) || !aligned(po, 16)) return ATTN_SINK_ERR_INVALID_ARG;
  return ATTN_SINK_OK;
}

// Ragged prefill: with pm == NULL the output goes to out (one chunk), else
// the partial states of num_splits chunks go to pm / pd / po.
int attn_sink_prefill_partials_impl(const void* q, const void* k, const void* v,
                                    const float* sinks, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_kv, int batch, int total_q,
                                    int total_kv, int max_seqlen_q, int num_kv_heads,
                                    int group_size, int head_dim, float sm_scale, int causal,
                                    int dtype, int num_splits, float* pm, float* pd, float* po,
                                    void* out, void* stream) {
  const int rc = check_prefill_common(q, sinks, cu_seqlens_q, batch, total_q, max_seqlen_q,
                                      num_kv_heads, group_size, head_dim, sm_scale, causal,
                                      dtype);
  if (rc != ATTN_SINK_OK) return rc;
  // k/v may be NULL only for an empty key set, out only for an empty query set
  if (!cu_seqlens_kv || ((!k || !v) && total_kv != 0) || total_kv < 0 ||
      (!pm && !out && total_q != 0))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(cu_seqlens_kv, 4))
    return ATTN_SINK_ERR_INVALID_ARG;
  const int es = dtype == ATTN_SINK_BF16 ? 2 : 4;
  if ((int64_t)total_kv * num_kv_heads * kHeadDim * es >= (int64_t)1 << 32 ||
      (int64_t)total_kv + (int64_t)kPage * num_splits > INT32_MAX)
    return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;
  PrefillArgs a{};
  a.q = (const char*)q;
  a.k = (const char*)k;
  a.v = (const char*)v;
  a.sinks = sinks;
  a.cu_q = cu_seqlens_q;
  a.cu_kv = cu_seqlens_kv;
  a.out = (char*)out;
  a.pm = pm;
  a.pd = pd;
  a.po = po;
  a.total_q = total_q;
  a.total_kv = total_kv;
  a.hkv = num_kv_heads;
  a.group = group_size;
  a.causal = causal;
  a.splits = num_splits;
  a.qk_scale_log2 = sm_scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return pm ? launch_prefill<false, true>(a, dtype, batch, max_seqlen_q, s)
            : launch_prefill<false, false>(a, dtype, batch, max_seqlen_q, s);
}

// Checks of the decode arguments other than the output buffers.
int check_decode_args(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* kv_lens, const float* sinks,
                      int batch, int max_pages_per_seq, int num_pages, int num_kv_heads,
                      int group_size, int head_dim, int page_size, float sm_scale, int dtype,
                      int num_splits) {
  // the caches may be NULL only when they hold no page
  if (!q || !page_table || !kv_lens || !sinks || ((!k_cache || !v_cache) && num_pages != 0))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (num_splits < 1) return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(page_table, 4) || !aligned(kv_lens, 4) || !aligned(sinks, 4))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (batch < 0 || max_pages_per_seq < 1 || num_pages < 0 || num_kv_heads < 1 ||
      group_size < 1 || head_dim < 1 || page_size < 1 ||
      (dtype != ATTN_SINK_F32 && dtype != ATTN_SINK_BF16) || !finite_positive(sm_scale))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kHeadDim || page_size != kPage || group_size > 16)
    return ATTN_SINK_ERR_UNSUPPORTED;
  if (batch > 65535 || num_kv_heads > 65535 ||
      (int64_t)max_pages_per_seq * kPage > INT32_MAX ||
      (int64_t)num_splits * max_pages_per_seq > INT32_MAX)
    return ATTN_SINK_ERR_UNSUPPORTED;
  return ATTN_SINK_OK;
}

int decode_paged_impl(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* page_table, const int32_t* kv_lens, const float* sinks,
                      int batch, int max_pages_per_seq, int num_pages, int num_kv_heads,
                      int group_size, int head_dim, int page_size, float sm_scale, int dtype,
                      int num_splits, float* partial_m, float* partial_d, float* partial_o,
                      void* out, void* stream) {
  const int rc = check_decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, batch,
                                   max_pages_per_seq, num_pages, num_kv_heads, group_size,
                                   head_dim, page_size, sm_scale, dtype, num_splits);
  if (rc != ATTN_SINK_OK) return rc;
  if (num_splits == 1 && !out) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_splits > 1 && (!partial_m || !partial_d || !partial_o)) return ATTN_SINK_ERR_INVALID_ARG;
  if ((out && !aligned(out, 16)) || (partial_m && !aligned(partial_m, 4)) ||
      (partial_d && !aligned(partial_d, 4)) || (partial_o && !aligned(partial_o, 16)))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (batch == 0) return ATTN_SINK_OK;
  const dim3 grid(num_splits, num_kv_heads, batch);
  const float qk = sm_scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
#define ATTN_SINK_DECODE(DTV, WV, UV)                                                          \
  hipLaunchKernelGGL((decode_kernel<DTV, WV, UV>), grid, dim3(64 * (WV)), 0, s,                 \
                     (const char*)q, (const char*)k_cache, (const char*)v_cache, page_table,   \
                     kv_lens, sinks, max_pages_per_seq, num_pages, num_kv_heads, group_size,   \
                     qk, num_splits, partial_m, partial_d, partial_o, (char*)out)
  // (fp32 page fragments are twice as large: at 16 waves, 128 VGPRs hold one
  // page group in flight per wave, not two)
  if (dtype == ATTN_SINK_BF16) {
    if (num_splits == 1) ATTN_SINK_DECODE(DT_BF16, kDecodeWavesUnsplit, kDecodeUnroll);
    else ATTN_SINK_DECODE(DT_BF16, kDecodeWaves, kDecodeUnroll);
  } else {
    if (num_splits == 1) ATTN_SINK_DECODE(DT_F32, kDecodeWavesUnsplit, 1);
    else ATTN_SINK_DECODE(DT_F32, kDecodeWaves, kDecodeUnroll);
  }
#undef ATTN_SINK_DECODE
  return launch_status();
}

int merge_impl(const float* partial_m, const float* partial_d, const float* partial_o,
               int batch, int num_q_heads, int num_splits, int head_dim, int out_dtype,
               void* out, void* stream) {
  if (!partial_m || !partial_d || !partial_o || !out) return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(partial_m, 4) || !aligned(partial_d, 4) || !aligned(partial_o, 16) ||
      !aligned(out, 16))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (batch < 0 || num_q_heads < 1 || num_splits < 1 || head_dim < 1 ||
      (out_dtype != ATTN_SINK_F32 && out_dtype != ATTN_SINK_BF16))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (head_dim != kHeadDim) return ATTN_SINK_ERR_UNSUPPORTED;
  const int64_t rows = (int64_t)batch * num_q_heads;
  if (rows > INT32_MAX - 16) return ATTN_SINK_ERR_UNSUPPORTED;
  if (rows == 0) return ATTN_SINK_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = out_dtype == ATTN_SINK_BF16;
  // Chunk lanes per row: the fewest that hold every chunk in registers (8
  // per thread), so that many rows take few workgroups -- each round of
  // workgroups costs one memory round trip -- but doubled while that leaves
  // fewer than about two workgroups per CU.  32768 rows in 4 splits: 10.5 us
  // with one lane per row against 17.6 with four; 4096 rows in 16 splits:
  // 8.0 against 11.4 with sixteen.  Past 128 chunks, 16 lanes and a second
  // loop.
  int cl = num_splits <= 8 ? 1 : num_splits <= 16 ? 2 : num_splits <= 32 ? 4
           : num_splits <= 64 ? 8 : 16;
  while (cl < 16 && rows * cl / 16 < 512) cl *= 2;
  const int rpb = 256 / (16 * cl);
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
#define ATTN_SINK_MERGE(CLV)                                                                  \
  hipLaunchKernelGGL((bf ? merge_kernel<DT_BF16, CLV> : merge_kernel<DT_F32, CLV>), grid,      \
                     dim3(256), 0, s, partial_m, partial_d, partial_o, (int)rows, num_splits,  \
                     (char*)out)
  switch (cl) {
    case 16: ATTN_SINK_MERGE(16); break;
    case 8: ATTN_SINK_MERGE(8); break;
    case 4: ATTN_SINK_MERGE(4); break;
    case 2: ATTN_SINK_MERGE(2); break;
    default: ATTN_SINK_MERGE(1); break;
  }
#undef ATTN_SINK_MERGE
  return launch_status();
}

// ------------------------------------------------- static scratch (no-alloc)
//
// attn_sink_decode_paged_static keeps its split partial states in this
// file-scope device array instead of caller- or library-allocated memory.
// Each GPU the library runs on holds its own copy until the process ends.
// In host code the array's name is only a host-side stand-in: its device
// address is resolved once per device with hipGetSymbolAddress (with that
// device current) and only that address is handed to kernels.

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
char* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the device `stream` belongs to.
int scratch_for(hipStream_t stream, char** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return ATTN_SINK_ERR_LAUNCH;
  int dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return ATTN_SINK_ERR_INVALID_ARG;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_SINK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return ATTN_SINK_ERR_LAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return ATTN_SINK_ERR_LAUNCH;
    if (e != hipSuccess || !p) return ATTN_SINK_ERR_LAUNCH;
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_SINK_OK;
}

}  // namespace

extern "C" {

const char* attn_sink_status_string(int status) {
  switch (status) {
    case ATTN_SINK_OK: return "ok";
    case ATTN_SINK_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_SINK_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_SINK_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_SINK_ERR_TOO_LARGE:
      return "split partial states exceed the 16 MiB static scratch buffer";
    default: return "unknown status";
  }
}

int attn_sink_prefill(const void* q, const void* k, const void* v, const float* sinks,
                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int batch,
                      int total_q, int total_kv, int max_seqlen_q, int num_kv_heads,
                      int group_size, int head_dim, float sm_scale, int causal, int dtype,
                      void* out, void* stream) {
  return attn_sink_prefill_partials_impl(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, batch,
                                         total_q, total_kv, max_seqlen_q, num_kv_heads,
                                         group_size, head_dim, sm_scale, causal, dtype, 1,
                                         nullptr, nullptr, nullptr, out, stream);
}

int attn_sink_prefill_partials(const void* q, const void* k, const void* v, const float* sinks,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                               int batch, int total_q, int total_kv, int max_seqlen_q,
                               int num_kv_heads, int group_size, int head_dim, float sm_scale,
                               int causal, int dtype, int num_splits, float* partial_m,
                               float* partial_d, float* partial_o, void* stream) {
  const int rc = check_partials(num_splits, partial_m, partial_d, partial_o);
  if (rc != ATTN_SINK_OK) return rc;
  return attn_sink_prefill_partials_impl(q, k, v, sinks, cu_seqlens_q, cu_seqlens_kv, batch,
                                         total_q, total_kv, max_seqlen_q, num_kv_heads,
                                         group_size, head_dim, sm_scale, causal, dtype,
                                         num_splits, partial_m, partial_d, partial_o, nullptr,
                                         stream);
}

int attn_sink_prefill_paged(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* cu_seqlens_q,
                            const int32_t* kv_lens, const float* sinks, int batch, int total_q,
                            int max_seqlen_q, int max_pages_per_seq, int num_pages,
                            int num_kv_heads, int group_size, int head_dim, int page_size,
                            float sm_scale, int causal, int dtype, int num_splits,
                            float* partial_m, float* partial_d, float* partial_o, void* out,
                            void* stream) {
  int rc = check_prefill_common(q, sinks, cu_seqlens_q, batch, total_q, max_seqlen_q,
                                num_kv_heads, group_size, head_dim, sm_scale, causal, dtype);
  if (rc != ATTN_SINK_OK) return rc;
  // the caches may be NULL only when they hold no page
  if (!page_table || !kv_lens || ((!k_cache || !v_cache) && num_pages != 0))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(page_table, 4) ||
      !aligned(kv_lens, 4))
    return ATTN_SINK_ERR_INVALID_ARG;
  if (num_splits == 1) {
    if ((!out && total_q != 0) || !aligned(out, 16)) return ATTN_SINK_ERR_INVALID_ARG;
  } else {
    rc = check_partials(num_splits, partial_m, partial_d, partial_o);
    if (rc != ATTN_SINK_OK) return rc;
  }
  if (max_pages_per_seq < 1 || num_pages < 0 || page_size < 1) return ATTN_SINK_ERR_INVALID_ARG;
  if (page_size != kPage) return ATTN_SINK_ERR_UNSUPPORTED;
  const int es = dtype == ATTN_SINK_BF16 ? 2 : 4;
  const int64_t cache_bytes = (int64_t)num_pages * num_kv_heads * kPage * kHeadDim * es;
  if ((int64_t)max_pages_per_seq * kPage + (int64_t)kPage * num_splits > INT32_MAX)
    return ATTN_SINK_ERR_UNSUPPORTED;
  // caches below 4 GiB: pages at 32-bit offsets from the cache base (buffer
  // loads); larger caches: 64-bit page bases
  const bool wide = cache_bytes >= (int64_t)1 << 32;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_SINK_OK;
  PrefillArgs a{};
  a.q = (const char*)q;
  a.k = (const char*)k_cache;
  a.v = (const char*)v_cache;
  a.sinks = sinks;
  a.cu_q = cu_seqlens_q;
  a.page_table = page_table;
  a.kv_lens = kv_lens;
  a.out = (char*)out;
  a.pm = partial_m;
  a.pd = partial_d;
  a.po = partial_o;
  a.total_q = total_q;
  a.hkv = num_kv_heads;
  a.group = group_size;
  a.causal = causal;
  a.splits = num_splits;
  a.max_pages = max_pages_per_seq;
  a.num_pages = num_pages;
  a.cache_bytes = wide ? 0u : (uint32_t)cache_bytes;
  a.qk_scale_log2 = sm_scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (wide)
    return num_splits == 1 ? launch_prefill<true, false, true>(a, dtype, batch, max_seqlen_q, s)
                           : launch_prefill<true, true, true>(a, dtype, batch, max_seqlen_q, s);
  return num_splits == 1 ? launch_prefill<true, false>(a, dtype, batch, max_seqlen_q, s)
                         : launch_prefill<true, true>(a, dtype, batch, max_seqlen_q, s);
}

int attn_sink_decode_paged(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* page_table, const int32_t* kv_lens, const float* sinks,
                           int batch, int max_pages_per_seq, int num_pages, int num_kv_heads,
                           int group_size, int head_dim, int page_size, float sm_scale,
                           int dtype, int num_splits, float* partial_m, float* partial_d,
                           float* partial_o, void* out, void* stream) {
  return decode_paged_impl(q, k_cache, v_cache, page_table, kv_lens, sinks, batch,
                           max_pages_per_seq, num_pages, num_kv_heads, group_size, head_dim,
                           page_size, sm_scale, dtype, num_splits, partial_m, partial_d,
                           partial_o, out, stream);
}

int attn_sink_merge(const float* partial_m, const float* partial_d, const float* partial_o,
                    int batch, int num_q_heads, int num_splits, int head_dim, int out_dtype,
                    void* out, void* stream) {
  return merge_impl(partial_m, partial_d, partial_o, batch, num_q_heads, num_splits, head_dim,
                    out_dtype, out, stream);
}

int attn_sink_decode_paged_static(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* page_table, const int32_t* kv_lens,
                                  const float* sinks, int batch, int max_pages_per_seq,
                                  int num_pages, int num_kv_heads, int group_size, int head_dim,
                                  int page_size, float sm_scale, int dtype, int num_splits,
                                  void* out, void* stream) {
  const int rc0 = check_decode_args(q, k_cache, v_cache, page_table, kv_lens, sinks, batch,
                                    max_pages_per_seq, num_pages, num_kv_heads, group_size,
                                    head_dim, page_size, sm_scale, dtype, num_splits);
  if (rc0 != ATTN_SINK_OK) return rc0;
  if (!out || !aligned(out, 16)) return ATTN_SINK_ERR_INVALID_ARG;
  if (num_splits == 1)
    return decode_paged_impl(q, k_cache, v_cache, page_table, kv_lens, sinks, batch,
                             max_pages_per_seq, num_pages, num_kv_heads, group_size, head_dim,
                             page_size, sm_scale, dtype, 1, nullptr, nullptr, nullptr, out,
                             stream);
  // partial states of (batch x Hq) rows x S chunks: m, d, then o, each
  // region 256-byte aligned inside the scratch array
  const int64_t states = (int64_t)batch * num_kv_heads * group_size * num_splits;
  const int64_t md_bytes = (states * 4 + 255) / 256 * 256;
  if (2 * md_bytes + states * kHeadDim * 4 > (int64_t)kScratchBytes) return ATTN_SINK_ERR_TOO_LARGE;
  if (batch == 0) return ATTN_SINK_OK;
  char* base = nullptr;
  const int rc = scratch_for(reinterpret_cast<hipStream_t>(stream), &base);
  if (rc != ATTN_SINK_OK) return rc;
  float* pm = reinterpret_cast<float*>(base);
  float* pd = reinterpret_cast<float*>(base + md_bytes);
  float* po = reinterpret_cast<float*>(base + 2 * md_bytes);
  const int rc2 = decode_paged_impl(q, k_cache, v_cache, page_table, kv_lens, sinks, batch,
                                    max_pages_per_seq, num_pages, num_kv_heads, group_size,
                                    head_dim, page_size, sm_scale, dtype, num_splits, pm, pd, po,
                                    nullptr, stream);
  if (rc2 != ATTN_SINK_OK) return rc2;
  return merge_impl(pm, pd, po, batch, num_kv_heads * group_size, num_splits, head_dim, dtype,
                    out, stream);
}

}  // extern "C"
