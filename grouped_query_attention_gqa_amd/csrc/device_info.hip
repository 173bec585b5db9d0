// gqa_device_info (declared in include/gqa.h): the compute-unit count and
// peak shader clock of a device, from which a measurement derives the
// roofline peaks of the board it ran on.  Kept apart from the launch code so
// that the measured kernels' sources do not change with it.

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "gqa.h"

extern "C" int32_t gqa_device_info(int32_t device, int32_t* compute_units, int32_t* max_clock_khz) {
  if (compute_units == nullptr || max_clock_khz == nullptr) return GQA_ERR_NULL;
  int cus = 0, khz = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device) != hipSuccess)
    return GQA_ERR_HIP;
  *compute_units = cus;
  *max_clock_khz = khz;
  return GQA_OK;
}
