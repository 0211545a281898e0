// Literal flags from byte content, on the host.
//
// "Parameter-free Adaptive Sparse Attention via Compression-Based Content
// Selection", Sec. 3.1 (Eq. 1 and Eq. 2) and Appendix B, Algorithm 1 steps 1-2:
// a sequence is cut into fixed-size blocks, each block is compressed on its own
// with gzip at level 1, and a block is literal when its compression ratio is
// above the sequence's mean ratio.  The ratio c_i / b and the mean
// (sum_j c_j) / (B b) are compared exactly in integers: c_i * B > sum_j c_j.
// The gzip container (10-byte header, 8-byte trailer) adds the same constant to
// every c_i, which the mean threshold cancels; it is kept so that c_i is the
// size gzip reports.
#include <stdint.h>
#include <string.h>
#include <zlib.h>

#include <vector>

#include "sparse_attn.h"

extern "C" sa_status sparse_attn_literal_flags(const uint8_t* bytes, int32_t G, int64_t n_bytes,
                                               int32_t block_bytes, int32_t level, uint8_t* flags_out,
                                               int32_t* sizes_out) {
  if (!bytes || !flags_out) return SA_ERR_NULL;
  if (G < 1 || n_bytes < 1 || block_bytes < 1 || level < 1 || level > 9) return SA_ERR_INVALID;
  if (n_bytes % block_bytes != 0) return SA_ERR_INVALID;
  const int64_t nb = n_bytes / block_bytes;
  if (nb > SA_MAX_BLOCKS) return SA_ERR_UNSUPPORTED;

  z_stream z;
  memset(&z, 0, sizeof(z));
  // window 15 with +16: gzip container; memory level 8 and the default
  // strategy are gzip's own settings
  if (deflateInit2(&z, level, Z_DEFLATED, 15 + 16, 8, Z_DEFAULT_STRATEGY) != Z_OK) return SA_ERR_INVALID;
  std::vector<unsigned char> out(deflateBound(&z, (uLong)block_bytes) + 64);
  std::vector<int64_t> sizes((size_t)nb);
  sa_status st = SA_OK;
  for (int32_t g = 0; g < G && st == SA_OK; ++g) {
    const uint8_t* seq = bytes + (int64_t)g * n_bytes;
    int64_t total = 0;
    for (int64_t i = 0; i < nb; ++i) {
      if (deflateReset(&z) != Z_OK) {
        st = SA_ERR_INVALID;
        break;
      }
      z.next_in = (Bytef*)(seq + i * block_bytes);
      z.avail_in = (uInt)block_bytes;
      z.next_out = out.data();
      z.avail_out = (uInt)out.size();
      if (deflate(&z, Z_FINISH) != Z_STREAM_END) {
        st = SA_ERR_INVALID;
        break;
      }
      sizes[(size_t)i] = (int64_t)z.total_out;
      total += sizes[(size_t)i];
    }
    if (st != SA_OK) break;
    for (int64_t i = 0; i < nb; ++i) {
      flags_out[(int64_t)g * nb + i] = sizes[(size_t)i] * nb > total ? 1 : 0;
      if (sizes_out) sizes_out[(int64_t)g * nb + i] = (int32_t)sizes[(size_t)i];
    }
  }
  deflateEnd(&z);
  return st;
}
