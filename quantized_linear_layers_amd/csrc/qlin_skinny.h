// Streaming core of the weight-bound ("skinny", M <= 64 rows) quantized
// GEMMs of libqlin: the dense decode GEMMs and the MoE expert GEMMs.
//
// A workgroup of NW waves (4 or 8) computes an (MB*16) x (NW * NB*16) output
// tile over one K range [k0, k1):
//  * activations pass through LDS in chunks of 256 K, double buffered and
//    shared by the NW waves (one barrier per chunk), fetched once per
//    workgroup in whole cache lines; K past the range is zeroed when
//    written; rows past the valid count are zeroed once, and waves whose
//    share of a chunk holds no valid row skip its loads and writes;
//  * each wave streams its own 16*NB weight rows in "units" (16 rows x 128
//    bytes per 16-row block: 128 K of fp8/int8, 256 K of int4 codes) with
//    line-shaped nontemporal loads (8 rows x 128 B per instruction), DEPTH
//    units ahead of use, and writes each unit to a wave-private LDS slot
//    from which the MFMA fragments are read (LDS operations of one wave
//    complete in order, so that slot needs no barrier);
//  * LDS blocks are "fragment-major": the 16 bytes that MFMA lane (r, g)
//    reads for one operand piece sit at piece*1024 + g*256 + 16*((r ^ c) & 15),
//    c being the 16-byte chunk of the row segment. The XOR keeps both access
//    shapes free of bank conflicts: a 16-byte LDS write is serviced 8 lanes
//    (128 bytes) at a time, and the 8 lanes of one staging write hold chunks
//    c = 0..7 of one row, so (r ^ c) & 7 takes 8 distinct values (r ^ 2c
//    would take 4: a 2-way conflict); the 16 lanes of a fragment read share
//    c and cover r = 0..15.
//      fp8 / int8 (2 KB per 16-row block and 128-K step): piece = K half h,
//        chunk c = 4h + g; weights use the same layout;
//      int4 weights (2 KB per block and unit of two steps): piece = step s,
//        chunk c = 4s + g (the 32 codes of group 4s + g);
//      bf16 activations (4 KB per block and step): piece = MFMA w of the
//        step, chunk c = 4g + w (values k = 32g + 8w .. +8).
//  * int4 group steps: with SB (16-byte aligned step rows, K % 256 == 0)
//    one 16-byte load per lane fetches the steps of 16 rows x DEPTH units
//    once per round of DEPTH units, into a wave-private LDS slot of DEPTH
//    units; otherwise each unit loads its own (4-byte granules of 2-byte
//    loads). Step slot layout: (unit * NB + j) * 256 + row * 16 + group * 2;
//  * the int4 unpack (bf16(c * step), exact product, one rounding, by
//    dequant8_mix) happens right before the MFMAs, after the activation
//    fragments of the same MFMAs are requested from LDS: scheduling barriers
//    keep the unpack between the two, so it covers the LDS latency (K=5120,
//    N=25600, M=64: 44.8 instead of 46.0 us; K=4096, N=14336, M=64: 32.7
//    instead of 37.9 us).
// Output layout: the weights are the MFMA's first operand, so acc[mb][j]
// register i of lane (r, g) is row mb*16 + r, column 16j + 4g + i of the
// wave's columns: each lane holds 4 consecutive columns of one row, which
// the epilogues store as one 8- or 16-byte piece.
#pragma once

#include <type_traits>

#include "qlin_device.h"
#include "qlin_internal.h"

namespace qlin {

template <int KIND>
using SkinnyAcc = typename std::conditional<KIND == kGemmI8, v4i, v4f>::type;

// Per-workgroup LDS bytes of skinny_mma<KIND, MB, NB, DEPTH, SB, NW, WK>.
template <int KIND, int MB, int NB, int DEPTH, int NW = 4, bool WK = false>
constexpr int skinny_lds_bytes() {
  return (WK ? NW : 1) * 2 * MB * 2 * 16 * 128 * (KIND == kGemmW4 ? 2 : 1) +
         NW * NB * (2048 + (KIND == kGemmW4 ? 256 * DEPTH : 0));
}

// Activation pieces (16 bytes) each thread stages per chunk: the chunk is
// split over the 64*NW threads of the workgroup, or with WK over the 64
// lanes of each wave.
template <int KIND, int MB, int NW, bool WK = false>
constexpr int skinny_pieces() {
  return MB * (KIND == kGemmW4 ? 2 : 1) * 4 / (WK ? 1 : NW);
}

// One weight unit of one wave in registers.
template <int KIND, int NB>
struct SkinnySlot {
  uint4 w[NB][2];
};
template <int NB>
struct SkinnySlot<kGemmW4, NB> {
  uint4 w[NB][2];
  uint32_t st[NB][2];
};

// Inputs of one tile, per lane:
//  wp[j][h]  weight row of block j, tile row 8h + lane/8, already offset by
//            16 * (lane % 8) bytes (clamped onto a valid row);
//  sp[j]     int4 group steps of tile row lane%16 of block j (W4A16 only);
//  wbytes    weight bytes per row (K or K/2);
//  ap[q]     activation row of this thread's chunk piece q (row
//            (tid + 64*NW*q) / (16 * ESZ) of the tile; clamped onto a valid row)
//  am[q]     0xFFFFFFFF if that row is a real row, else 0 (the real rows
//            must be a prefix of the tile's rows);
//  K         full K (clamps the activation loads), k0/k1 the range.
// WK: every wave has its own K range [k0, k1) (the arguments differ per
// wave) and stages its own activation chunks in a wave-private LDS region
// (no workgroup barriers inside; LDS operations of one wave complete in
// order). The caller sums the waves' accumulators.
template <int KIND, int MB, int NB, int DEPTH, bool SB = false, int NW = 4, bool WK = false>
__device__ __forceinline__ void skinny_mma(uint8_t* lds, const uint8_t* (&wp)[NB][2], const uint16_t* (&sp)[NB],
                                           const uint8_t* (&ap)[skinny_pieces<KIND, MB, NW, WK>()],
                                           uint32_t (&am)[skinny_pieces<KIND, MB, NW, WK>()], int K, int k0,
                                           int k1, SkinnyAcc<KIND> (&acc)[MB][NB]) {
  constexpr bool W4 = KIND == kGemmW4;
  constexpr int ESZ = W4 ? 2 : 1;                    // activation bytes per element
  constexpr int kUnitK = W4 ? 256 : 128;             // K per weight unit
  constexpr int UPC = 256 / kUnitK;                  // units per activation chunk
  static_assert(DEPTH % (2 * UPC) == 0, "a round holds an even number of chunks");
  constexpr int kBlk = 16 * 128 * ESZ;               // LDS bytes per (mb, step) of activations
  constexpr int kBuf = MB * 2 * kBlk;                // one 256-K activation chunk
  constexpr int kRowPieces = 16 * ESZ;               // 16-byte pieces per row per chunk
  constexpr int NT = WK ? 64 : 64 * NW;              // threads staging one activation chunk
  constexpr int kPer = skinny_pieces<KIND, MB, NW, WK>();  // activation pieces per thread per chunk
  static_assert(kPer * NT == MB * ESZ * 256 && kPer >= 1, "activation chunk split over the threads");
  constexpr int kWSlot = NB * 2048;                  // one wave's weight unit in LDS
  constexpr int kSSlot = W4 ? DEPTH * NB * 256 : 0;  // ... and its int4 group steps
  static_assert(!SB || (W4 && DEPTH <= 4), "bulk steps: W4A16, one load covers <= 4 units");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int tid = WK ? lane : (int)threadIdx.x;      // index among the staging threads
  const int r = lane & 15, g = lane >> 4;
  const int nunits = (k1 - k0 + kUnitK - 1) / kUnitK;
  constexpr int kActs = (WK ? NW : 1) * 2 * kBuf;    // activation region
  uint8_t* const act = lds + (WK ? wave * 2 * kBuf : 0);
  uint8_t* wslot = lds + kActs + wave * kWSlot;
  uint8_t* sslot = lds + kActs + NW * kWSlot + wave * kSSlot;
  auto block_sync = [&]() {
    if constexpr (!WK) __syncthreads();
  };

  // ---- weights
  const int wc = lane & 7;
  const int bclamp = (W4 ? k1 / 2 : k1) - 16 - 16 * wc;
  const int gmax = k1 / 32 - 1;
  auto wload = [&](SkinnySlot<KIND, NB>& sl, int u) {
    const int kb = k0 + u * kUnitK;
    const int bo = min(W4 ? kb / 2 : kb, bclamp);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      sl.w[j][0] = ldg16_nt(wp[j][0] + bo);
      sl.w[j][1] = ldg16_nt(wp[j][1] + bo);
      if constexpr (W4 && !SB) {
        const int gi = kb / 32 + 2 * (lane >> 4);
        sl.st[j][0] = sp[j][min(gi, gmax)];
        sl.st[j][1] = sp[j][min(gi + 1, gmax)];
      }
    }
  };
  const int wr = (wc >> 2) * 1024 + (wc & 3) * 256;
  auto wstage = [&](const SkinnySlot<KIND, NB>& sl) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int R = 8 * h + (lane >> 3);
        *reinterpret_cast<uint4*>(wslot + j * 2048 + wr + ((R ^ wc) & 15) * 16) = sl.w[j][h];
      }
      if constexpr (W4 && !SB)
        *reinterpret_cast<uint32_t*>(sslot + j * 256 + (lane & 15) * 16 + (lane >> 4) * 4) =
            (sl.st[j][0] & 0xFFFFu) | (sl.st[j][1] << 16);
    }
  };

  // ---- bulk int4 steps (SB): lane (row lane%16, unit lane/16 % DEPTH) of
  // the round of DEPTH units starting at unit u0; past the range: clamped
  // onto the row's last 16 bytes, never used
  const int su = (lane >> 4) & (DEPTH - 1);
  const int spmax = k1 / 256 - 1;
  uint4 sreg[NB];
  auto sload = [&](int u0) {
    if constexpr (SB) {
      const int pc = min(k0 / 256 + u0 + su, spmax);
#pragma unroll
      for (int j = 0; j < NB; ++j) sreg[j] = ldg16(sp[j] + 8 * pc);
    }
  };
  auto swrite = [&]() {
    if constexpr (SB) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        *reinterpret_cast<uint4*>(sslot + (su * NB + j) * 256 + (lane & 15) * 16) = sreg[j];
    }
  };

  // ---- activation chunks. Loads are clamped and stay unmasked in
  // registers (masking them at load time would make the next instruction
  // wait for every load in flight); the mask is applied by the LDS write.
  // qv[q]: this wave's share of piece q holds a valid row (uniform: the
  // wave's first row is valid, and valid rows are a prefix). Only the
  // W4A16 path skips the others (4x the activation traffic per weight
  // byte); for fp8/int8 the branches cost more registers than they save.
  // register sets of activation chunks in flight: two (chunk ci + 2 loaded
  // at the start of chunk ci) for fp8/int8, one (chunk ci + 1) for W4A16,
  // whose bf16 chunks take twice the registers
  constexpr int kSets = W4 ? 1 : 2;
  uint4 aset[kSets][kPer];
  bool qv[kPer];
#pragma unroll
  for (int q = 0; q < kPer; ++q) qv[q] = !W4 || __builtin_amdgcn_readfirstlane(am[q]) != 0u;
  auto aoff = [&](int q, int buf) {
    const int pc = tid + NT * q;
    const int row = pc / kRowPieces, piece = pc % kRowPieces;
    const int mb = row >> 4, rr = row & 15;
    const int s = piece / (8 * ESZ), c = piece % (8 * ESZ);
    int off;
    if constexpr (W4) off = (c & 3) * 1024 + (c >> 2) * 256 + ((rr ^ c) & 15) * 16;
    else off = (c >> 2) * 1024 + (c & 3) * 256 + ((rr ^ c) & 15) * 16;
    return (int)(act - lds) + buf * kBuf + (mb * 2 + s) * kBlk + off;
  };
  auto aload = [&](int ci, uint4 (&dst)[kPer]) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (qv[q]) {
        const int piece = (tid + NT * q) % kRowPieces;
        const int k = k0 + ci * 256 + piece * (16 / ESZ);
        dst[q] = ldg16(ap[q] + (size_t)min(k, K - 16 / ESZ) * ESZ);
      }
    }
  };
  auto awrite = [&](const uint4 (&src)[kPer], int ci, int buf) {
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
      if (qv[q]) {
        const int piece = (tid + NT * q) % kRowPieces;
        const int k = k0 + ci * 256 + piece * (16 / ESZ);
        const uint32_t m = k < k1 ? am[q] : 0u;
        uint4 v = src[q];
        *reinterpret_cast<uint4*>(lds + aoff(q, buf)) = make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
      }
    }
  };
  const int rd0 = g * 256 + ((r ^ g) & 15) * 16;
  const int rd1 = 1024 + g * 256 + ((r ^ (4 + g)) & 15) * 16;
  const int rdw = g * 256;

  // multiply the weight unit in the wave's slot (unit u) with the
  // activation chunk that holds it
  auto compute = [&](int u, int d) {
    const uint8_t* abase = act + ((u / UPC) & 1) * kBuf;
    if constexpr (W4) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        uint4 cw[NB];
        Int4Step st[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          cw[j] = *reinterpret_cast<const uint4*>(wslot + j * 2048 + s * 1024 + g * 256 +
                                                  ((r ^ (4 * s + g)) & 15) * 16);
          st[j] = int4_step(bf16_f32(*reinterpret_cast<const uint16_t*>(sslot + ((SB ? d : 0) * NB + j) * 256 +
                                                                        r * 16 + (4 * s + g) * 2)));
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // the step's activation fragments are requested first, so that
          // the unpack below runs while they are in flight
          const int off = s * kBlk + w * 1024 + rdw + ((r ^ (4 * g + w)) & 15) * 16;
          v8bf af[MB];
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) af[mb] = *reinterpret_cast<const v8bf*>(abase + mb * 2 * kBlk + off);
          __builtin_amdgcn_sched_barrier(0);
          v8bf bf[NB];
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const uint32_t word = w == 0 ? cw[j].x : w == 1 ? cw[j].y : w == 2 ? cw[j].z : cw[j].w;
            bf[j] = dequant8_mix(word, st[j]);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[mb][j] = mfma_bf16(bf[j], af[mb], acc[mb][j]);
        }
      }
    } else {
      const uint8_t* ab = abase + (u & 1) * kBlk;
      v4i w0[NB], w1[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        w0[j] = *reinterpret_cast<const v4i*>(wslot + j * 2048 + rd0);
        w1[j] = *reinterpret_cast<const v4i*>(wslot + j * 2048 + rd1);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const v4i a0 = *reinterpret_cast<const v4i*>(ab + mb * 2 * kBlk + rd0);
        const v4i a1 = *reinterpret_cast<const v4i*>(ab + mb * 2 * kBlk + rd1);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          if constexpr (KIND == kGemmFP8) {
            acc[mb][j] = mfma_fp8(__builtin_shufflevector(w0[j], w1[j], 0, 1, 2, 3, 4, 5, 6, 7),
                                  __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7), acc[mb][j]);
          } else {
            acc[mb][j] = mfma_i8(w0[j], a0, acc[mb][j]);
            acc[mb][j] = mfma_i8(w1[j], a1, acc[mb][j]);
          }
        }
      }
    }
  };

  // ---- prologue: steps of the first round, activation chunks 0 and 1 in
  // registers, chunk 0 in LDS, padding rows of both buffers zeroed, the
  // weight ring filled
  sload(0);
  aload(0, aset[0]);
  if constexpr (kSets == 2) aload(1, aset[1]);
  SkinnySlot<KIND, NB> ring[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) wload(ring[d], d);
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    if (!qv[q]) {
      *reinterpret_cast<uint4*>(lds + aoff(q, 0)) = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(lds + aoff(q, 1)) = make_uint4(0, 0, 0, 0);
    }
  }
  awrite(aset[0], 0, 0);
  block_sync();

  // ---- main loop over whole rounds of DEPTH units. Activation chunk ci
  // uses LDS buffer ci & 1 and register set ci % kSets; at its start the
  // set is refilled with chunk ci + kSets, after its last unit chunk ci + 1
  // goes to the other buffer. Each unit: its registers go to the wave's slot, the ring
  // slot is refilled DEPTH units ahead (past the range: clamped loads of
  // valid memory, never used), then the unit is multiplied. The scheduling
  // barriers keep each refill right after the write that freed its slot.
  // With SB the round's steps go to the step slot first and the next
  // round's are loaded (the step slot is read only by this wave, in order).
  const int full = nunits / DEPTH, rem = nunits % DEPTH;
  for (int rd = 0; rd < full; ++rd) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int u = rd * DEPTH + d;
      if (d % UPC == 0) aload(u / UPC + kSets, aset[(d / UPC) % kSets]);
      if (d == 0) {
        swrite();
        sload(u + DEPTH);
      }
      wstage(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
      wload(ring[d], u + DEPTH);
      __builtin_amdgcn_sched_barrier(0);
      compute(u, d);
      if (d % UPC == UPC - 1) {
        awrite(aset[((d / UPC) + 1) % kSets], u / UPC + 1, (u / UPC + 1) & 1);
        block_sync();
      }
    }
  }
  // ---- the last rem units are already in the ring; the activation chunks
  // continue as above (their steps are in sreg). The condition is uniform
  // over the workgroup.
  if (rem > 0) swrite();
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    if (d < rem) {
      const int u = full * DEPTH + d;
      if (d % UPC == 0) aload(u / UPC + kSets, aset[(d / UPC) % kSets]);
      wstage(ring[d]);
      compute(u, d);
      if (d % UPC == UPC - 1 && d + 1 < rem) {
        awrite(aset[((d / UPC) + 1) % kSets], u / UPC + 1, (u / UPC + 1) & 1);
        block_sync();
      }
    }
  }
}

}  // namespace qlin
