/*
 * ceiling.h - measurement kernels of libceiling.so (not part of the loss):
 * the HBM rate of the Dr. GRPO row kernel's access pattern with no
 * arithmetic, and the device's properties, for benchmark reports.
 */
#ifndef CEILING_H
#define CEILING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { CEILING_COPY = 0, CEILING_FILL = 1, CEILING_READ = 2 };

/* One 1024-thread workgroup per row of row_bytes (a multiple of 16, at most
 * 311,296), workgroup b on row (b * row_stride) mod rows, all of a row's
 * 16-byte loads in flight before its stores (nontemporal loads, sc1|nt
 * buffer stores), as the loss's row kernel moves a vocabulary row.
 *   CEILING_COPY  src row -> dst row; with row_read (nullable, [rows] device
 *                 bytes) rows flagged 0 are only written with zeros
 *   CEILING_FILL  zeros -> dst row
 *   CEILING_READ  src row read; sink ([rows] uint32, device) is written
 *                 only for a row whose words XOR to one fixed value
 * src, dst 16-byte aligned device pointers; stream a hipStream_t; ev_begin /
 * ev_end optional hipEvent_t stamped by the dispatch itself.  Returns 0, or
 * -1 (NULL), -2 (sizes), -3 (mode), -6 (alignment), -7 (launch failed). */
int ceiling_rows(const void* src, void* dst, int64_t rows, int64_t row_bytes, int64_t row_stride,
                 int32_t mode, const uint8_t* row_read, uint32_t* sink, void* stream,
                 void* ev_begin, void* ev_end);

/* The loss's active / zero row mix in its ticket order: as CEILING_COPY
 * with row_read, but workgroup b takes the class (row_read flag) of row
 * (b * row_stride) mod rows and then the next row of that class in memory
 * order: class_rows ([rows] uint32, device) lists the n_read flagged rows in
 * increasing order, then the others in increasing order; counters ([65]
 * uint32, device) holds the two classes' tickets at [0] and [64], zeroed by
 * the call on `stream` before the timed dispatch.  Flags, class_rows and
 * n_read must agree (a workgroup whose ticket runs past its class does
 * nothing).  Returns as ceiling_rows, -1 also for a NULL row_read,
 * class_rows or counters and -2 for n_read outside [0, rows]. */
int ceiling_rows_ticket(const void* src, void* dst, int64_t rows, int64_t row_bytes,
                        int64_t row_stride, const uint8_t* row_read, const uint32_t* class_rows,
                        int64_t n_read, uint32_t* counters, void* stream, void* ev_begin,
                        void* ev_end);

/* Properties of device `device` (hipGetDeviceProperties and the runtime's
 * versions).  Returns 0, -1 (NULL) or -7. */
typedef struct ceiling_device_info {
  char name[256];
  char arch[256];
  int32_t compute_units;
  int32_t clock_khz;         /* maximum shader clock */
  int32_t memory_clock_khz;
  int32_t memory_bus_bits;
  int64_t total_mem_bytes;
  int32_t l2_bytes;
  int32_t runtime_version;
  int32_t driver_version;
} ceiling_device_info_t;

int ceiling_device_info(int device, ceiling_device_info_t* out);

#ifdef __cplusplus
}
#endif

#endif /* CEILING_H */
