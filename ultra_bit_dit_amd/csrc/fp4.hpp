// fp4 (e2m1) operands from the packed weight layout, shared by the GEMV and
// GEMM kernels (internal, not part of the public ABI).
//
// A lane L = r + 16q of a wavefront owns row r of a 16-row block and quarter
// q of each 128-weight group; its 32 weights of a group decode into the four
// fp4 registers of operand B of v_mfma_scale_f32_16x16x128_f8f6f4 (nibble s
// of the 128-bit operand = slot s): +1 = 0x2, -1 = 0xA, 0 = 0x0.
#pragma once

#include "common.hpp"

namespace lowbit {

typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));

// packed codes of one quad (4 groups) of one lane, and its 4 fp16 scales
template <int FMT>
struct Quad {
  u4 w[FMT == 1 ? 1 : 2];  // binary: 4 words; 2-bit: P0/P1 of 2 groups per vector
  u2 c30, c31, c32;        // base-3: 24 bytes of 5-trit bytes
  uint32_t t3;             // base-3: the two 4-trit bytes of this quad
  uint2 sc;
};

// Codes and scales of quad gq of row-block rb for lane L (unconditional
// loads: callers clamp rb and gq into the matrix).  pscales NULL reads any
// readable memory instead (unit scales are applied by the caller).
template <int FMT>
__device__ __attribute__((always_inline)) inline void load_quad_at(const uint8_t* pcodes,
                                                                  const uint16_t* pscales,
                                                                  int64_t rb, int64_t gq,
                                                                  int64_t GQ, int64_t GP,
                                                                  int L, Quad<FMT>& o) {
  const int r = L & 15;
  const u4* pcv = (const u4*)pcodes;
  if constexpr (FMT == 1) {
    o.w[0] = __builtin_nontemporal_load(&pcv[(rb * GQ + gq) * 64 + L]);
  } else if constexpr (FMT == 3) {
    // octet block (rb, gq/2): plane s of lane L at 1024 s + 16 L; the quad's
    // half h = gq % 2 takes 8-byte chunks 3h .. 3h+2 (chunk c = plane c/2,
    // half c%2) and bytes 2h, 2h+1 of the 4-byte word at 3072 + 4 L
    const int64_t GO = cdiv(GQ, 2);
    const uint8_t* ob = pcodes + (rb * GO + (gq >> 1)) * 3328;
    const int h = (int)(gq & 1);
    const uint8_t* lp = ob + 16 * L;
    o.c30 = __builtin_nontemporal_load((const u2*)(lp + (h ? 1024 + 8 : 0)));
    o.c31 = __builtin_nontemporal_load((const u2*)(lp + (h ? 2048 : 8)));
    o.c32 = __builtin_nontemporal_load((const u2*)(lp + (h ? 2048 + 8 : 1024)));
    o.t3 = __builtin_nontemporal_load((const uint32_t*)(ob + 3072 + 4 * L)) >> (16 * h);
  } else {
    const int64_t p0 = 2 * gq, p1 = min<int64_t>(2 * gq + 1, GP - 1);
    o.w[0] = __builtin_nontemporal_load(&pcv[(rb * GP + p0) * 64 + L]);
    o.w[1] = __builtin_nontemporal_load(&pcv[(rb * GP + p1) * 64 + L]);
  }
  const uint2* sbase = pscales ? (const uint2*)pscales : (const uint2*)pcodes;
  o.sc = sbase[(rb * GQ + gq) * 16 + r];
}

// base-3: byte value -> its 5 trits as fp4 nibbles (trit 0 -> -1 = 0xA,
// 1 -> 0, 2 -> +1 = 0x2), nibble e = trit e (least significant first)
__device__ __attribute__((always_inline)) inline uint32_t trit_nibbles(uint32_t v) {
  uint32_t nib = 0;
#pragma unroll
  for (int e = 0; e < 5; e++) {
    const uint32_t t = v % 3;
    v /= 3;
    nib |= (t == 0 ? 0xAu : t == 2 ? 0x2u : 0u) << (4 * e);
  }
  return nib;
}

// The table of trit_nibbles in LDS, TS copies interleaved: entry v of copy c
// at word TS v + c.  Lane L reads copy L % TS, so a wave's 64 random lookups
// spread over the banks instead of colliding on the 243 words of a single
// copy.  Threads of a block of `nthreads` fill it together.
template <int TS = 1>
__device__ __attribute__((always_inline)) inline void fill_trit_table(uint32_t* t3, int nthreads = 256) {
  static_assert(TS == 1 || TS % 4 == 0, "copies are written four at a time");
  for (int e = threadIdx.x; e < 243; e += nthreads) {
    const uint32_t nib = trit_nibbles((uint32_t)e);
    if constexpr (TS == 1) {
      t3[e] = nib;
    } else {
#pragma unroll
      for (int c = 0; c < TS; c += 4) *(uint4*)(t3 + TS * e + c) = make_uint4(nib, nib, nib, nib);
    }
  }
}

// bytes of the LDS table with TS copies
constexpr int trit_table_bytes(int ts) { return 243 * 4 * ts <= 1024 ? 1024 : 243 * 4 * ts; }

// fp16 scale of group t of a quad
template <int FMT>
__device__ __attribute__((always_inline)) inline float quad_scale(const Quad<FMT>& qd, int t) {
  return f16_bits_to_f32((t < 2 ? qd.sc.x : qd.sc.y) >> (16 * (t & 1)));
}

// fp4 operand B of group t of a quad (base-3: t3 is the lane's copy of a
// table with TS interleaved copies, i.e. the table plus L % TS)
template <int FMT, int TS = 1>
__device__ __attribute__((always_inline)) inline v8i decode_group(const Quad<FMT>& qd, int t,
                                                                  const uint32_t* t3) {
  uint32_t d0, d1, d2, d3;
  if constexpr (FMT == 1) {
    const u4 c4 = qd.w[0];
    const uint32_t wv = t == 0 ? c4.x : t == 1 ? c4.y : t == 2 ? c4.z : c4.w;
    d0 = (wv & 0x88888888u) | 0x22222222u;
    d1 = ((wv << 1) & 0x88888888u) | 0x22222222u;
    d2 = ((wv << 2) & 0x88888888u) | 0x22222222u;
    d3 = ((wv << 3) & 0x88888888u) | 0x22222222u;
  } else if constexpr (FMT == 3) {
    // group t of the quad: bytes 6t .. 6t+5 hold slots 0..29, the 4-trit
    // byte t/2 digits 2(t%2), 2(t%2)+1 hold slots 30, 31
    auto word = [&](int wi) {
      return wi == 0 ? qd.c30.x : wi == 1 ? qd.c30.y : wi == 2 ? qd.c31.x
           : wi == 3 ? qd.c31.y : wi == 4 ? qd.c32.x : qd.c32.y;
    };
    uint32_t nb[6];
#pragma unroll
    for (int i = 0; i < 6; i++) {
      const int byte = 6 * t + i;
      nb[i] = t3[TS * ((word(byte >> 2) >> (8 * (byte & 3))) & 0xFFu)];
    }
    const uint32_t tl = (t3[TS * ((qd.t3 >> (8 * (t >> 1))) & 0xFFu)] >> (8 * (t & 1))) & 0xFFu;
    // slot s -> nibble s of d0..d3 (5 slots per byte)
    const uint64_t lo = (uint64_t)nb[0] | ((uint64_t)nb[1] << 20) | ((uint64_t)nb[2] << 40) |
                        ((uint64_t)nb[3] << 60);
    const uint64_t hi = (uint64_t)(nb[3] >> 4) | ((uint64_t)nb[4] << 16) |
                        ((uint64_t)nb[5] << 36) | ((uint64_t)tl << 56);
    d0 = (uint32_t)lo;
    d1 = (uint32_t)(lo >> 32);
    d2 = (uint32_t)hi;
    d3 = (uint32_t)(hi >> 32);
  } else {
    const u4 c4 = qd.w[t >> 1];
    const uint32_t p0 = (t & 1) ? c4.z : c4.x, p1 = (t & 1) ? c4.w : c4.y;
    d0 = p0 & 0xAAAAAAAAu;
    d1 = (p0 << 1) & 0xAAAAAAAAu;
    d2 = p1 & 0xAAAAAAAAu;
    d3 = (p1 << 1) & 0xAAAAAAAAu;
  }
  return v8i{(int)d0, (int)d1, (int)d2, (int)d3, 0, 0, 0, 0};
}

// fp4 operand B of binary group t with the two masks held in registers
// (a VOP3 instruction takes no literal here): one v_and_or_b32 for slot
// register 0 and a shift plus v_and_or_b32 for each of the other three.
__device__ __attribute__((always_inline)) inline v8i decode_binary_reg(uint32_t wv, uint32_t sign_mask,
                                                                       uint32_t one_bits) {
  const uint32_t d0 = (wv & sign_mask) | one_bits;
  const uint32_t d1 = ((wv << 1) & sign_mask) | one_bits;
  const uint32_t d2 = ((wv << 2) & sign_mask) | one_bits;
  const uint32_t d3 = ((wv << 3) & sign_mask) | one_bits;
  return v8i{(int)d0, (int)d1, (int)d2, (int)d3, 0, 0, 0, 0};
}

}  // namespace lowbit
