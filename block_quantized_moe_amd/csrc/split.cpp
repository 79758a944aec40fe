// Host-side loader split: on-disk (array-of-structs) quant blocks -> the
// GPU-resident struct-of-arrays tensors the kernels read.
//
// The GGUF block-dequant page ("Design -- CPU-side decomposition") splits each
// on-disk block once at load time into separate GPU-resident tensors (packed
// codes, scales, lookup tables) so the hot kernels do no per-call byte
// surgery; the DSV4 campaign page repacks q2_K blocks to SoA at load because
// the AoS code bytes sit at 84*blk+16 and are only 4-byte aligned.  Here every
// output array is naturally aligned and contiguous per block.
#include <stdint.h>
#include <string.h>

#include "../../include/qmoe.h"

extern "C" {

int qmoe_split_q8_0(const void* aos, int64_t n_blocks, int8_t* qs, uint16_t* d) {
  if (!aos || !qs || !d || n_blocks < 0) return QMOE_ERR_ARG;
  const uint8_t* p = (const uint8_t*)aos;
  for (int64_t b = 0; b < n_blocks; ++b, p += 34) {
    memcpy(&d[b], p, 2);
    memcpy(&qs[b * 32], p + 2, 32);
  }
  return QMOE_OK;
}

int qmoe_split_q2_k(const void* aos, int64_t n_blocks, uint32_t* qs, uint8_t* scales,
                    uint16_t* d, uint16_t* dmin) {
  if (!aos || !qs || !scales || !d || !dmin || n_blocks < 0) return QMOE_ERR_ARG;
  const uint8_t* p = (const uint8_t*)aos;
  for (int64_t b = 0; b < n_blocks; ++b, p += 84) {
    memcpy(&scales[b * 16], p, 16);
    memcpy(&qs[b * 16], p + 16, 64);  // 16 little-endian u32 words
    memcpy(&d[b], p + 80, 2);
    memcpy(&dmin[b], p + 82, 2);
  }
  return QMOE_OK;
}

int qmoe_split_iq2_xxs(const void* aos, int64_t n_blocks, uint32_t* idx, uint32_t* aux,
                       uint16_t* d) {
  if (!aos || !idx || !aux || !d || n_blocks < 0) return QMOE_ERR_ARG;
  const uint8_t* p = (const uint8_t*)aos;
  for (int64_t b = 0; b < n_blocks; ++b, p += 66) {
    memcpy(&d[b], p, 2);
    for (int g = 0; g < 8; ++g) {
      memcpy(&idx[b * 8 + g], p + 2 + 8 * g, 4);
      memcpy(&aux[b * 8 + g], p + 2 + 8 * g + 4, 4);
    }
  }
  return QMOE_OK;
}

int qmoe_split_int4(const uint32_t* words, int64_t n_words, uint32_t* out) {
  if (!words || !out || n_words < 0) return QMOE_ERR_ARG;
  for (int64_t w = 0; w < n_words; ++w) {
    const uint32_t v = words[w];
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
      r |= ((v >> (8 * i)) & 0xFu) << (4 * i);            // element 2i   -> nibble i
      r |= ((v >> (8 * i + 4)) & 0xFu) << (4 * i + 16);   // element 2i+1 -> nibble 4+i
    }
    out[w] = r;
  }
  return QMOE_OK;
}

void qmoe_iq2_signs_table(uint8_t out[128]) {
  if (!out) return;
  for (int i = 0; i < 128; ++i) {
    const int odd = __builtin_popcount((unsigned)i) & 1;
    out[i] = (uint8_t)(i | (odd << 7));
  }
}

}  // extern "C"
