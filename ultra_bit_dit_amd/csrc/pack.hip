// Pack / unpack between dense codes + fp16 scales and the gfx950 layout.
//
// Each packed word is produced by one thread that gathers its 32 (binary) or
// 16 (2-bit) codes, or its 52 base-3 bytes, straight from the dense matrix;
// every dense code is read by exactly one thread, so invalid codes are
// counted once.  One-time work (not on the timed path).
#include "common.hpp"

namespace lowbit {
namespace {

__device__ inline int dense_code(const int8_t* codes, int64_t N, int64_t K, int64_t n,
                                 int64_t k, bool pad) {
  if (pad || n >= N || k >= K) return 0;
  return codes[n * K + k];
}

__device__ inline void count_bad(int32_t* bad, int nbad) {
  if (!bad) return;
  // one atomic per wave
  unsigned long long ball = __ballot(nbad != 0);
  if (ball == 0) return;
  int tot = nbad;
  for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
  if ((threadIdx.x & 63) == __ffsll(ball) - 1) atomicAdd(bad, tot);
}

// ---------------------------------------------------------------- binary
__global__ void pack_binary(int64_t N, int64_t K, int64_t GQ, int64_t nwords,
                            const int8_t* __restrict__ codes, uint32_t* __restrict__ out,
                            int32_t* bad) {
  int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int nbad = 0;
  if (wi < nwords) {
    int t = wi & 3, L = (wi >> 2) & 63;
    int64_t blk = wi >> 8, rb = blk / GQ, gq = blk % GQ;
    int64_t g = 4 * gq + t, n = 16 * rb + (L & 15);
    int q = L >> 4;
    bool pad = g * kGroup >= K;
    uint32_t w = 0;
    for (int b = 0; b < 32; b++) {
      int c = dense_code(codes, N, K, n, g * kGroup + kmap(q, bin_slot(b)), pad);
      if (!pad && n < N && c != 1 && c != -1) nbad++;
      w |= (uint32_t)(c == -1) << b;
    }
    out[wi] = w;
  }
  count_bad(bad, nbad);
}

__global__ void unpack_binary(int64_t N, int64_t K, int64_t GQ, int64_t nwords,
                              const uint32_t* __restrict__ in, int8_t* __restrict__ codes) {
  int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= nwords) return;
  int t = wi & 3, L = (wi >> 2) & 63;
  int64_t blk = wi >> 8, rb = blk / GQ, gq = blk % GQ;
  int64_t g = 4 * gq + t, n = 16 * rb + (L & 15);
  int q = L >> 4;
  if (n >= N || g * kGroup >= K) return;
  uint32_t w = in[wi];
  for (int b = 0; b < 32; b++)
    codes[n * K + g * kGroup + kmap(q, bin_slot(b))] = ((w >> b) & 1) ? -1 : 1;
}

// ------------------------------------------------------------ ternary 2-bit
__global__ void pack_tern2(int64_t N, int64_t K, int64_t GP, int64_t nwords,
                           const int8_t* __restrict__ codes, uint32_t* __restrict__ out,
                           int32_t* bad) {
  int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int nbad = 0;
  if (wi < nwords) {
    int t = wi & 1, gg = (wi >> 1) & 1, L = (wi >> 2) & 63;
    int64_t blk = wi >> 8, rb = blk / GP, gp = blk % GP;
    int64_t g = 2 * gp + gg, n = 16 * rb + (L & 15);
    int q = L >> 4;
    bool pad = g * kGroup >= K;
    uint32_t w = 0;
    for (int jj = 0; jj < 2; jj++)
      for (int p = 0; p < 8; p++) {
        int i = 8 * (2 * t + jj) + p;
        int c = dense_code(codes, N, K, n, g * kGroup + kmap(q, i), pad);
        if (c < -1 || c > 1) {
          if (!pad && n < N) nbad++;
          c = 0;
        }
        w |= (uint32_t)(c != 0) << (4 * p + 1 - jj);
        w |= (uint32_t)(c < 0) << (4 * p + 3 - jj);
      }
    out[wi] = w;
  }
  count_bad(bad, nbad);
}

__global__ void unpack_tern2(int64_t N, int64_t K, int64_t GP, int64_t nwords,
                             const uint32_t* __restrict__ in, int8_t* __restrict__ codes,
                             int32_t* bad) {
  int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int nbad = 0;
  if (wi < nwords) {
    int t = wi & 1, gg = (wi >> 1) & 1, L = (wi >> 2) & 63;
    int64_t blk = wi >> 8, rb = blk / GP, gp = blk % GP;
    int64_t g = 2 * gp + gg, n = 16 * rb + (L & 15);
    int q = L >> 4;
    if (n < N && g * kGroup < K) {
      uint32_t w = in[wi];
      for (int jj = 0; jj < 2; jj++)
        for (int p = 0; p < 8; p++) {
          int i = 8 * (2 * t + jj) + p;
          int z = (w >> (4 * p + 1 - jj)) & 1, sg = (w >> (4 * p + 3 - jj)) & 1;
          int c = z ? (sg ? -1 : 1) : 0;
          if (!z && sg) nbad++;
          codes[n * K + g * kGroup + kmap(q, i)] = (int8_t)c;
        }
    }
  }
  count_bad(bad, nbad);
}

// ------------------------------------------------------------ ternary base-3
// byte index / digit of slot i of group j (0..7) inside a lane's 52 bytes
__device__ inline void b3_pos(int j, int i, int& byte, int& digit) {
  if (i < 30) {
    byte = 6 * j + i / 5;
    digit = i % 5;
  } else {
    byte = 48 + j / 2;
    digit = 2 * (j & 1) + (i - 30);
  }
}

__device__ inline int64_t b3_addr(int64_t blk, int L, int b) {
  return blk * 3328 + (b < 48 ? 1024 * (b >> 4) + 16 * L + (b & 15) : 3072 + 4 * L + (b - 48));
}

__global__ void pack_tern3(int64_t N, int64_t K, int64_t GO, int64_t nlanes,
                           const int8_t* __restrict__ codes, uint8_t* __restrict__ out,
                           int32_t* bad) {
  int64_t li = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int nbad = 0;
  if (li < nlanes) {
    int L = li & 63;
    int64_t blk = li >> 6, rb = blk / GO, o = blk % GO;
    int64_t n = 16 * rb + (L & 15);
    int q = L >> 4;
    int B[52];
    for (int b = 0; b < 52; b++) B[b] = 0;
    const int pw3[5] = {1, 3, 9, 27, 81};
    for (int j = 0; j < 8; j++) {
      int64_t g = 8 * o + j;
      bool pad = g * kGroup >= K;
      for (int i = 0; i < 32; i++) {
        int c = dense_code(codes, N, K, n, g * kGroup + kmap(q, i), pad);
        if (c < -1 || c > 1) {
          if (!pad && n < N) nbad++;
          c = 0;
        }
        int byte, digit;
        b3_pos(j, i, byte, digit);
        B[byte] += (c + 1) * pw3[digit];
      }
    }
    // 3 x 16 bytes + 4 bytes, little-endian words
    uint32_t wv[13];
    for (int w = 0; w < 13; w++)
      wv[w] = (uint32_t)B[4 * w] | ((uint32_t)B[4 * w + 1] << 8) | ((uint32_t)B[4 * w + 2] << 16) |
              ((uint32_t)B[4 * w + 3] << 24);
    for (int s = 0; s < 3; s++) {
      uint4 v = make_uint4(wv[4 * s], wv[4 * s + 1], wv[4 * s + 2], wv[4 * s + 3]);
      *(uint4*)(out + b3_addr(blk, L, 16 * s)) = v;
    }
    *(uint32_t*)(out + b3_addr(blk, L, 48)) = wv[12];
  }
  count_bad(bad, nbad);
}

__global__ void unpack_tern3(int64_t N, int64_t K, int64_t GO, int64_t nlanes,
                             const uint8_t* __restrict__ in, int8_t* __restrict__ codes,
                             int32_t* bad) {
  int64_t li = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int nbad = 0;
  if (li < nlanes) {
    int L = li & 63;
    int64_t blk = li >> 6, rb = blk / GO, o = blk % GO;
    int64_t n = 16 * rb + (L & 15);
    int q = L >> 4;
    if (n < N) {
      for (int j = 0; j < 8; j++) {
        int64_t g = 8 * o + j;
        if (g * kGroup >= K) break;
        for (int i = 0; i < 32; i++) {
          int byte, digit;
          b3_pos(j, i, byte, digit);
          int v = in[b3_addr(blk, L, byte)];
          int c;
          if (v >= (byte < 48 ? 243 : 81)) {
            nbad++;
            c = 0;
          } else {
            for (int d = 0; d < digit; d++) v /= 3;
            c = v % 3 - 1;
          }
          codes[n * K + g * kGroup + kmap(q, i)] = (int8_t)c;
        }
      }
    }
  }
  count_bad(bad, nbad);
}

// ---------------------------------------------------------------- scales
__global__ void pack_scales(int64_t N, int64_t G, int64_t GQ, int64_t nslots,
                            const uint16_t* __restrict__ scales, uint16_t* __restrict__ out) {
  int64_t si = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= nslots) return;
  int t = si & 3, r = (si >> 2) & 15;
  int64_t blk = si >> 6, rb = blk / GQ, gq = blk % GQ;
  int64_t g = 4 * gq + t, n = 16 * rb + r;
  out[si] = (n < N && g < G) ? scales[n * G + g] : (uint16_t)0;
}

__global__ void unpack_scales(int64_t N, int64_t G, int64_t GQ, int64_t nslots,
                              const uint16_t* __restrict__ in, uint16_t* __restrict__ scales) {
  int64_t si = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (si >= nslots) return;
  int t = si & 3, r = (si >> 2) & 15;
  int64_t blk = si >> 6, rb = blk / GQ, gq = blk % GQ;
  int64_t g = 4 * gq + t, n = 16 * rb + r;
  if (n < N && g < G) scales[n * G + g] = in[si];
}

inline dim3 grid_for(int64_t n, int block) { return dim3((unsigned)cdiv(n, block)); }

}  // namespace

hipError_t launch_pack(int fmt, int64_t N, int64_t K, const int8_t* codes,
                       const uint16_t* scales, void* pcodes, void* pscales, int32_t* bad,
                       hipStream_t s) {
  const int B = 256;
  int64_t NB = cdiv(N, 16), G = K / kGroup, GQ = cdiv(G, 4);
  if (fmt == 1) {
    int64_t nw = NB * GQ * 256;
    hipLaunchKernelGGL(pack_binary, grid_for(nw, B), dim3(B), 0, s, N, K, GQ, nw, codes,
                       (uint32_t*)pcodes, bad);
  } else if (fmt == 2) {
    int64_t GP = cdiv(G, 2), nw = NB * GP * 256;
    hipLaunchKernelGGL(pack_tern2, grid_for(nw, B), dim3(B), 0, s, N, K, GP, nw, codes,
                       (uint32_t*)pcodes, bad);
  } else {
    int64_t GO = cdiv(G, 8), nl = NB * GO * 64;
    hipLaunchKernelGGL(pack_tern3, grid_for(nl, B), dim3(B), 0, s, N, K, GO, nl, codes,
                       (uint8_t*)pcodes, bad);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t ns = NB * GQ * 64;
  hipLaunchKernelGGL(pack_scales, grid_for(ns, B), dim3(B), 0, s, N, G, GQ, ns, scales,
                     (uint16_t*)pscales);
  return hipGetLastError();
}

hipError_t launch_unpack(int fmt, int64_t N, int64_t K, const void* pcodes,
                         const void* pscales, int8_t* codes, uint16_t* scales, int32_t* bad,
                         hipStream_t s) {
  const int B = 256;
  int64_t NB = cdiv(N, 16), G = K / kGroup, GQ = cdiv(G, 4);
  if (fmt == 1) {
    int64_t nw = NB * GQ * 256;
    hipLaunchKernelGGL(unpack_binary, grid_for(nw, B), dim3(B), 0, s, N, K, GQ, nw,
                       (const uint32_t*)pcodes, codes);
  } else if (fmt == 2) {
    int64_t GP = cdiv(G, 2), nw = NB * GP * 256;
    hipLaunchKernelGGL(unpack_tern2, grid_for(nw, B), dim3(B), 0, s, N, K, GP, nw,
                       (const uint32_t*)pcodes, codes, bad);
  } else {
    int64_t GO = cdiv(G, 8), nl = NB * GO * 64;
    hipLaunchKernelGGL(unpack_tern3, grid_for(nl, B), dim3(B), 0, s, N, K, GO, nl,
                       (const uint8_t*)pcodes, codes, bad);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t ns = NB * GQ * 64;
  hipLaunchKernelGGL(unpack_scales, grid_for(ns, B), dim3(B), 0, s, N, G, GQ, ns,
                     (const uint16_t*)pscales, scales);
  return hipGetLastError();
}

}  // namespace lowbit
