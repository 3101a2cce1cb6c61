// placeholder, filled in by the backward kernels
#include "vsa_device.h"
